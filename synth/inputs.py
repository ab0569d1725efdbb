"""Seeded generator for paged block-sparse attention inputs.

Recipe (applies to every workload below):

* block = page = 128 tokens; pools are head-major per page ("HND"):
  K, V ``[P, Hkv, 128, D]`` and index-K ``[P, Hidx, 128, Di]``.
* Values are float32 N(0,1) draws rounded to the storage type with
  round-to-nearest-even (bf16 / f32), or, for fp8-e4m3 pools, divided by the
  per-tensor scale, clamped to +-448 and rounded to e4m3fn.  MX-fp4 pools
  (OCP E2M1 codes with an E8M0 scale per 32 elements) hold, per (page,
  head), the 128 x D / 2 code bytes then the 128 x D / 32 scale bytes of the
  draws divided by the per-tensor scale: per group of 32 the scale is
  2^(floor(log2 max|x|) - 2) and each code the nearest E2M1 value of
  x / scale (ties to the even code, clamped at 6).
* Physical page ids come from a seeded permutation; ``P`` = pages used plus
  ``max(8, ceil(1%))`` spare pages.  Unused block-table entries are -1.
* Poison: spare pages and the token slots past ``seq_len`` in every
  sequence's last page hold NaN in K/V (bf16 0x7FC0, f32 NaN, fp8 0x7F) and
  +1e4 in index-K, so that any read of an invalid slot shows up in results.
* Sequence lengths drawn at random come from a CPU ``torch.Generator``
  seeded with ``seed``, so they are the same whichever device generates the
  case.  Everything else is drawn, in the order permutation, q, idx_q, K, V,
  idx_K (then idx_V, for workloads with the index-value branch), from one
  generator on ``device`` seeded with ``seed``; pools are drawn in chunks of
  256 pages.  CPU and GPU draws of those differ; every
  consumer gets the bytes of one draw.

Decode: one query per sequence at position ``seq_len - 1``.  Prefill: the
``n_new`` new tokens of a sequence are its last ones, at positions
``seq_len - n_new .. seq_len - 1``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK = 128
PAGE_CHUNK = 256

# The workloads the library is measured and checked on, by shape.
WORKLOADS = {
    "decode_b2_l2048": dict(
        kind="decode", B=2, seq_lens=("fixed", 2048), Hq=8, Hkv=1, Hidx=1,
        D=128, Di=64, topk=4, init=1, local=2, q="bf16", kv="bf16", idx="bf16"),
    "decode_b32_l32k": dict(
        kind="decode", B=32, seq_lens=("fixed", 32768), Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=16, init=1, local=2, q="bf16", kv="bf16", idx="bf16"),
    "decode_b64_lvar": dict(
        kind="decode", B=64, seq_lens=("uniform", 4096, 131072), Hq=16, Hkv=2,
        Hidx=2, D=128, Di=128, topk=32, init=1, local=2, q="bf16", kv="bf16",
        idx="bf16"),
    "prefill_4x4096_p16k": dict(
        kind="prefill", B=4, n_new=4096, prefix=16384, Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=16, init=1, local=2, q="bf16", kv="bf16", idx="bf16"),
    "decode_fp8_b32_l64k": dict(
        kind="decode", B=32, seq_lens=("fixed", 65536), Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=32, init=1, local=2, q="bf16", kv="fp8", idx="bf16",
        k_scale=1.0 / 16, v_scale=1.0 / 16),
    # multi-token decode (speculative verification): 4 new tokens per sequence
    "verify_b32_q4_l32k": dict(
        kind="prefill", B=32, n_new=4, prefix=32764, Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=16, init=1, local=2, q="bf16", kv="bf16", idx="bf16"),
    # paged append of a 4 x 4096-token chunk into pools of 4 x 20480 tokens
    # (the step before the path; slots in a seeded random order)
    "append_4x4096": dict(
        kind="append", T=16384, pool_tokens=4 * 20480, Hq=16, Hkv=2, Hidx=2, D=128,
        Di=128, topk=16, init=1, local=2, q="bf16", kv="bf16", idx="bf16"),
    "append_fp8_4x4096": dict(
        kind="append", T=16384, pool_tokens=4 * 20480, Hq=16, Hkv=2, Hidx=2, D=128,
        Di=128, topk=16, init=1, local=2, q="bf16", kv="fp8", idx="bf16",
        k_scale=1.0 / 16, v_scale=1.0 / 16),
    # fp8-e5m2 K/V pools (the other fp8 cache format of the sglang page)
    "decode_e5m2_b32_l64k": dict(
        kind="decode", B=32, seq_lens=("fixed", 65536), Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=32, init=1, local=2, q="bf16", kv="fp8_e5m2", idx="bf16",
        k_scale=1.0 / 16, v_scale=1.0 / 16),
    # the index-value branch on (an index-value pool beside the index keys)
    "decode_iv_b32_l32k": dict(
        kind="decode", B=32, seq_lens=("fixed", 32768), Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=16, init=1, local=2, q="bf16", kv="bf16", idx="bf16",
        idx_value=True),
    "prefill_iv_4x4096_p16k": dict(
        kind="prefill", B=4, n_new=4096, prefix=16384, Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=16, init=1, local=2, q="bf16", kv="bf16", idx="bf16",
        idx_value=True),
    # MX-fp4 K/V pools (4-bit codes with a scale per 32 elements): the fp8
    # decode workload's shape
    "decode_mxfp4_b32_l64k": dict(
        kind="decode", B=32, seq_lens=("fixed", 65536), Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=32, init=1, local=2, q="bf16", kv="mxfp4", idx="bf16"),
    # MX-fp6 (E2M3) K/V pools, same shape
    "decode_mxfp6_b32_l64k": dict(
        kind="decode", B=32, seq_lens=("fixed", 65536), Hq=16, Hkv=2, Hidx=2,
        D=128, Di=128, topk=32, init=1, local=2, q="bf16", kv="mxfp6", idx="bf16"),
}

# Seeds of the workloads, in the order above.
WORKLOAD_SEEDS = {name: 1001 + i for i, name in enumerate(WORKLOADS)}

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn,
             "fp8_e5m2": torch.float8_e5m2}
MX_GROUP = 32


def mxfp4_run_bytes(D: int) -> int:
    return BLOCK * D // 2 + BLOCK * D // MX_GROUP


def _mxfp4_runs(y: torch.Tensor) -> torch.Tensor:
    """[n, H, 128, D] float32 -> [n, H, run bytes] uint8 (codes, then scales)."""
    n, H, T, D = y.shape
    g = y.reshape(n, H, T, D // MX_GROUP, MX_GROUP)
    amax = g.abs().amax(dim=-1)
    _, e = torch.frexp(amax)
    k = torch.where(amax > 0, e - 3, torch.full_like(e, -127))
    sc = (k + 127).clamp(0, 254)
    a = torch.ldexp(g, (127 - sc).unsqueeze(-1)).abs()
    code = ((a > 0.25).to(torch.int32) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
            + (a >= 3.5) + (a > 5.0))
    code = (code | (torch.signbit(g).to(torch.int32) << 3)).reshape(n, H, T, D)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    return torch.cat([packed.reshape(n, H, -1), sc.to(torch.uint8).reshape(n, H, -1)], dim=-1)


def mxfp6_run_bytes(D: int) -> int:
    return BLOCK * D * 3 // 4 + BLOCK * D // MX_GROUP


def _mxfp6_runs(y: torch.Tensor) -> torch.Tensor:
    """[n, H, 128, D] float32 -> [n, H, run bytes] uint8: E2M3 codes packed four
    to three bytes (element i of a 32-group at bits 6 i of its 24 bytes, little
    endian), then the E8M0 scales."""
    n, H, T, D = y.shape
    g = y.reshape(n, H, T, D // MX_GROUP, MX_GROUP)
    amax = g.abs().amax(dim=-1)
    _, e = torch.frexp(amax)
    k = torch.where(amax > 0, e - 3, torch.full_like(e, -127))
    sc = (k + 127).clamp(0, 254)
    a = torch.ldexp(g, (127 - sc).unsqueeze(-1)).abs().clamp(max=7.5)
    step = torch.where(a < 2.0, 0.125, torch.where(a < 4.0, 0.25, 0.5))
    v = torch.round(a / step) * step                      # half to even
    code = torch.where(v < 2.0, v * 8, torch.where(v < 4.0, 8 + v * 4, 16 + v * 2))
    code = (code.to(torch.int32) | (torch.signbit(g).to(torch.int32) << 5)).reshape(n, H, T, D // 4, 4)
    w = code[..., 0] | (code[..., 1] << 6) | (code[..., 2] << 12) | (code[..., 3] << 18)
    packed = torch.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], dim=-1).to(torch.uint8)
    return torch.cat([packed.reshape(n, H, -1), sc.to(torch.uint8).reshape(n, H, -1)], dim=-1)


_MX_RUN_BYTES = {"mxfp4": mxfp4_run_bytes, "mxfp6": mxfp6_run_bytes}
_MX_RUNS = {"mxfp4": _mxfp4_runs, "mxfp6": _mxfp6_runs}
_POISON_KV = {"bf16": float("nan"), "f32": float("nan"), "mxfp4": 0.0, "mxfp6": 0.0}
FP8_NAN_BYTE = 0x7F
IDX_POISON = 1.0e4


def workload(name: str, **overrides) -> dict:
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    spec["name"] = name
    return spec


@dataclasses.dataclass
class Case:
    spec: dict
    seq_lens: torch.Tensor          # [B] int32
    cu_seqlens_q: Optional[torch.Tensor]  # [B+1] int32 (prefill) or None (decode)
    block_table: torch.Tensor       # [B, MB] int32, -1 padded
    q: torch.Tensor                 # [T, Hq, D]
    idx_q: torch.Tensor             # [T, Hidx, Di]
    k_pool: torch.Tensor            # [P, Hkv, 128, D] (fp8 pools are uint8)
    v_pool: torch.Tensor
    idx_k_pool: torch.Tensor        # [P, Hidx, 128, Di]
    num_pages: int
    k_scale: float = 1.0
    v_scale: float = 1.0
    idx_v_pool: Optional[torch.Tensor] = None  # [P, Hidx, 128, Di] (index-value branch)

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def to(self, device) -> "Case":
        f = {}
        for fld in dataclasses.fields(self):
            v = getattr(self, fld.name)
            f[fld.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Case(**f)


def _draw_seq_lens(spec, seed) -> torch.Tensor:
    B = spec["B"]
    if spec["kind"] == "prefill":
        n_new = spec["n_new"]
        n_new = list(n_new) if isinstance(n_new, Sequence) else [n_new] * B
        prefix = spec["prefix"]
        prefix = list(prefix) if isinstance(prefix, Sequence) else [prefix] * B
        return torch.tensor([a + b for a, b in zip(prefix, n_new)], dtype=torch.int32)
    sl = spec["seq_lens"]
    if isinstance(sl, (list, tuple)) and sl and sl[0] == "fixed":
        return torch.full((B,), int(sl[1]), dtype=torch.int32)
    if isinstance(sl, (list, tuple)) and sl and sl[0] == "uniform":
        lo, hi = int(sl[1]), int(sl[2])
        g = torch.Generator(device="cpu")
        g.manual_seed(int(seed))
        return torch.randint(lo, hi + 1, (B,), generator=g).to(torch.int32)
    return torch.tensor(list(sl), dtype=torch.int32)


def _quantise(x: torch.Tensor, dtype: str, scale: float) -> torch.Tensor:
    if dtype == "fp8":
        y = (x / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        return y.view(torch.uint8)
    if dtype == "fp8_e5m2":
        y = (x / scale).clamp_(-57344.0, 57344.0).to(torch.float8_e5m2)
        return y.view(torch.uint8)
    return x.to(_TORCH_DT[dtype])


def _draw_pool(P, H, Dm, dtype, scale, g, device) -> torch.Tensor:
    if dtype in _MX_RUNS:
        pool = torch.empty((P, H, _MX_RUN_BYTES[dtype](Dm)), dtype=torch.uint8, device=device)
    else:
        out_dt = torch.uint8 if dtype.startswith("fp8") else _TORCH_DT[dtype]
        pool = torch.empty((P, H, BLOCK, Dm), dtype=out_dt, device=device)
    for p0 in range(0, P, PAGE_CHUNK):
        p1 = min(P, p0 + PAGE_CHUNK)
        x = torch.randn((p1 - p0, H, BLOCK, Dm), generator=g, device=device,
                        dtype=torch.float32)
        if dtype in _MX_RUNS:
            pool[p0:p1] = _MX_RUNS[dtype](x / scale)
        else:
            pool[p0:p1] = _quantise(x, dtype, scale)
    return pool


def _poison(pool: torch.Tensor, valid: torch.Tensor, dtype: str, value: float):
    """Overwrite token slots ``t >= valid[page]`` of every page."""
    tok = torch.arange(BLOCK, device=pool.device)
    bad = tok[None, :] >= valid.to(pool.device)[:, None]          # [P,128]
    if dtype in _MX_RUNS:
        # the NaN scale code (0xFF) for every group of the slot; the run is
        # 128 D / 2 (fp4) or 128 D 3 / 4 (fp6) code bytes, then 128 D / 32 scales
        per_d = BLOCK // 2 if dtype == "mxfp4" else BLOCK * 3 // 4
        D = pool.shape[-1] // (per_d + BLOCK // MX_GROUP)
        nsc = D // MX_GROUP
        sc = pool[:, :, pool.shape[-1] - BLOCK * nsc:].view(pool.shape[0], pool.shape[1], BLOCK, nsc)
        sc.masked_fill_(bad[:, None, :, None].expand(sc.shape), 0xFF)
        return
    bad = bad[:, None, :, None].expand(pool.shape)
    if dtype.startswith("fp8"):
        pool.masked_fill_(bad, FP8_NAN_BYTE)   # NaN in e4m3 and in e5m2
    else:
        pool.masked_fill_(bad, value)


def generate(spec: dict, seed: int, device="cpu", max_blocks: Optional[int] = None,
             poison: bool = True, spare_pages: Optional[int] = None) -> Case:
    """Draw one seeded case of ``spec`` on ``device`` (see the module recipe)."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    B, Hq, Hkv, Hidx = spec["B"], spec["Hq"], spec["Hkv"], spec["Hidx"]
    D, Di = spec["D"], spec["Di"]
    qd, kvd, idd = spec.get("q", "bf16"), spec.get("kv", "bf16"), spec.get("idx", "bf16")
    k_scale = float(spec.get("k_scale", 1.0))
    v_scale = float(spec.get("v_scale", 1.0))

    # 1. sequence lengths
    seq_lens = _draw_seq_lens(spec, seed)
    nb = [(int(L) + BLOCK - 1) // BLOCK for L in seq_lens.tolist()]
    used = sum(nb)
    spare = spare_pages if spare_pages is not None else max(8, math.ceil(used / 100))
    P = used + spare
    MB = max(nb) if nb else 1
    if max_blocks is not None:
        if max_blocks < MB:
            raise ValueError("max_blocks smaller than the longest sequence")
        MB = max_blocks
    MB = max(MB, 1)

    # 2. page permutation -> block table
    perm = torch.randperm(P, generator=g, device=device).to(torch.int32).cpu()
    bt = torch.full((B, MB), -1, dtype=torch.int32)
    valid = torch.zeros(P, dtype=torch.int32)
    off = 0
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(nb[b]):
            page = int(perm[off + j])
            bt[b, j] = page
            valid[page] = min(BLOCK, L - j * BLOCK)
        off += nb[b]

    if spec["kind"] == "prefill":
        n_new = spec["n_new"]
        n_new = list(n_new) if isinstance(n_new, Sequence) else [n_new] * B
        cu = torch.zeros(B + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(n_new, dtype=torch.int32), 0)
        T = int(cu[-1])
    else:
        cu = None
        T = B

    # 3-4. queries
    q = torch.randn((T, Hq, D), generator=g, device=device).to(_TORCH_DT[qd])
    idx_q = torch.randn((T, Hidx, Di), generator=g, device=device).to(_TORCH_DT[idd])

    # 5-7. pools
    k_pool = _draw_pool(P, Hkv, D, kvd, k_scale, g, device)
    v_pool = _draw_pool(P, Hkv, D, kvd, v_scale, g, device)
    idx_k_pool = _draw_pool(P, Hidx, Di, idd, 1.0, g, device)
    idx_v_pool = _draw_pool(P, Hidx, Di, idd, 1.0, g, device) if spec.get("idx_value") else None

    if poison:
        _poison(k_pool, valid, kvd, _POISON_KV.get(kvd, 0.0))
        _poison(v_pool, valid, kvd, _POISON_KV.get(kvd, 0.0))
        _poison(idx_k_pool, valid, idd, IDX_POISON)
        if idx_v_pool is not None:
            _poison(idx_v_pool, valid, idd, _POISON_KV.get(idd, 0.0))

    return Case(spec=dict(spec), seq_lens=seq_lens.to(device),
                cu_seqlens_q=None if cu is None else cu.to(device),
                block_table=bt.to(device), q=q, idx_q=idx_q, k_pool=k_pool,
                v_pool=v_pool, idx_k_pool=idx_k_pool, num_pages=P,
                k_scale=k_scale, v_scale=v_scale, idx_v_pool=idx_v_pool)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def host_view(case: Case, pages: Optional[np.ndarray] = None) -> dict:
    """Raw host copies of a case's bytes, tagged with their storage types.

    bf16 tensors come back as uint16 bit patterns, fp8 pools as uint8 codes,
    f32 as float32.  ``pages`` (optional) copies only those physical pages of
    the pools; the others are left as zero-filled placeholders, which keeps
    host memory bounded when only a few sequences are checked.
    """
    spec = case.spec

    def pool(t):
        if pages is None:
            return _bits(t)
        host = np.zeros(tuple(t.shape), dtype=_bits(t[:1]).dtype)
        idx = torch.as_tensor(np.asarray(pages, dtype=np.int64), device=t.device)
        host[np.asarray(pages, dtype=np.int64)] = _bits(t.index_select(0, idx))
        return host

    return dict(
        q=_bits(case.q), idx_q=_bits(case.idx_q),
        k_pool=pool(case.k_pool), v_pool=pool(case.v_pool),
        idx_k_pool=pool(case.idx_k_pool),
        idx_v_pool=None if case.idx_v_pool is None else pool(case.idx_v_pool),
        block_table=_bits(case.block_table), seq_lens=_bits(case.seq_lens),
        cu_seqlens_q=None if case.cu_seqlens_q is None else _bits(case.cu_seqlens_q),
        q_dtype=spec.get("q", "bf16"), kv_dtype=spec.get("kv", "bf16"),
        idx_dtype=spec.get("idx", "bf16"),
        k_scale=case.k_scale, v_scale=case.v_scale,
        topk=spec["topk"], init=spec["init"], local=spec["local"],
        forced_in_budget=bool(spec.get("forced_in_budget", False)),
        score_type=spec.get("score_type", "max"),
        Hq=spec["Hq"], Hkv=spec["Hkv"], Hidx=spec["Hidx"],
    )
