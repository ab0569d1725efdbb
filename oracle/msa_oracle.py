"""fp64 CPU oracle for block-sparse attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module; the library's product
path never does, and this module imports nothing from the library.

What is computed (plain definitions, no blocking, fusion or split):

* Sources.  The sglang page ``minimax_sparse_backend.py``
  (``MiniMaxSparseAttnBackend.__init__``) derives ``init_blocks``,
  ``local_blocks`` and ``topk_blocks`` for a per-token selection
  (``block_size_q = 1``, ``block_size_k`` = 128) and hands the index-head
  query/keys to the sparse decode/prefill ops; the vLLM page
  ``sparse_attention_msa.py`` (``MiniMaxM3SparseMSAImpl.forward``) runs
  causal attention (``causal=True``) over the selected 128-token KV blocks of
  a paged cache, with fp8 K/V scales (``k_scale``/``v_scale``).  The score
  type is left open by the pages; the reading used here is: a block's score
  is the maximum over its visible tokens of ``q_idx . k_idx``, and equal
  scores go to the lower block index.

* Every floating-point value is decoded exactly to float64 first (bf16 by
  its bit layout, fp8-e4m3fn through a table built from the format
  definition); all arithmetic after that is float64.

Readings of the pages taken here (each also recorded with the design notes):

* top-k is drawn from the blocks that are not forced, and the result is the
  union with the forced init and local blocks (|S| = min(nb, |F| + topk));
* local blocks are the trailing ``local`` blocks ending at the query's own,
  possibly partial, block; init blocks are the first ``init`` blocks;
* tokens after the query position are invisible both to scoring and to
  attention; decode attends to its own (already written) token;
* head maps: q head ``hq`` reads kv head ``hq // (Hq/Hkv)``; kv head ``g``
  uses index head ``g // (Hkv/Hidx)``;
* selections are listed in ascending block order, -1 padded.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

BLOCK = 128


# --------------------------------------------------------------------------
# Exact decoding of stored values
# --------------------------------------------------------------------------

def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of an IEEE binary32: shift the 16 stored
    bits into the high half of a 32-bit word and reinterpret."""
    u32 = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def fp8_e4m3fn_table() -> np.ndarray:
    """Values of the 256 OCP FP8 E4M3 ("e4m3fn") codes.

    Layout s.eeee.mmm, exponent bias 7; exponent field 0 encodes subnormals
    m/8 * 2^-6; no infinities; s.1111.111 is NaN.  The vLLM page's query
    dequantisation notes that every E4M3 value is exact in bf16.
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = math.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


def fp8_e5m2_table() -> np.ndarray:
    """Values of the 256 OCP FP8 E5M2 codes.

    Layout s.eeeee.mm, exponent bias 15; exponent field 0 encodes subnormals
    m/4 * 2^-14; exponent field 31 encodes +-inf (m = 0) and NaN (m != 0), as
    in IEEE binary16, of which E5M2 is the top byte.  The sglang page keeps
    fp8 main caches in this format, as in E4M3, on its sparse path that
    dequantises on load.
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 2) & 0x1F
        m = code & 0x3
        if e == 0x1F:
            tab[code] = sign * math.inf if m == 0 else math.nan
        elif e == 0:
            tab[code] = sign * (m / 4.0) * 2.0 ** (1 - 15)
        else:
            tab[code] = sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return tab


_FP8_TABLE = None
_E5M2_TABLE = None


def decode(arr: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Stored representation -> float64 values (times ``scale`` for fp8)."""
    global _FP8_TABLE, _E5M2_TABLE
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        if _FP8_TABLE is None:
            _FP8_TABLE = fp8_e4m3fn_table()
        return _FP8_TABLE[np.asarray(arr, dtype=np.uint8)] * float(scale)
    if dtype == "fp8_e5m2":
        if _E5M2_TABLE is None:
            _E5M2_TABLE = fp8_e5m2_table()
        return _E5M2_TABLE[np.asarray(arr, dtype=np.uint8)] * float(scale)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Query positions
# --------------------------------------------------------------------------

def query_positions(seq_lens: np.ndarray, cu_seqlens_q: Optional[np.ndarray],
                    positions=None):
    """List of (sequence b, position p) per query token.

    Decode (no cu_seqlens_q): one query per sequence at p = L_b - 1.
    Prefill: the n_b = cu[b+1]-cu[b] new tokens are the sequence's last ones,
    p = L_b - n_b + i (the sglang page passes prefix lengths alongside
    ``cu_seqlens``; the prefix is L_b - n_b).  ``positions`` (a list of
    (b, p)) names the query rows explicitly instead, e.g. a sample of a
    prefill's tokens.
    """
    if positions is not None:
        return [(int(b), int(p)) for b, p in positions]
    out = []
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if cu_seqlens_q is None:
        for b, L in enumerate(seq_lens):
            out.append((b, int(L) - 1))
    else:
        cu = np.asarray(cu_seqlens_q, dtype=np.int64)
        for b, L in enumerate(seq_lens):
            n = int(cu[b + 1] - cu[b])
            for i in range(n):
                out.append((b, int(L) - n + i))
    return out


def num_visible_blocks(p: int) -> int:
    """Blocks holding at least one token t <= p."""
    return 0 if p < 0 else p // BLOCK + 1


# --------------------------------------------------------------------------
# Step 1: block scores from the index heads
# --------------------------------------------------------------------------

# Block score types.  The sglang page reads a score type from the model
# config and hands it to the sparse ops without printing its values; "max" is
# the reading the spec fixes.  Two other reductions over a block's visible
# tokens are offered beside it (names and definitions of this library):
#   "mean": the mean of q_idx . k_idx (equivalently q_idx . the mean visible
#           key of the block);
#   "lse":  log sum exp(q_idx . k_idx / sqrt(Di)), the block's share of a
#           softmax over the index logits, in the log domain.
SCORE_TYPES = ("max", "mean", "lse")


def reduce_block(dots: np.ndarray, score_type: str, Di: int) -> float:
    """One block's score from the dots of its visible tokens (non-empty)."""
    if score_type == "max":
        return float(np.max(dots))
    if score_type == "mean":
        return float(np.mean(dots))
    if score_type == "lse":
        z = dots / math.sqrt(Di)
        m = float(np.max(z))
        return m + math.log(float(np.sum(np.exp(z - m))))
    raise ValueError(score_type)


def block_scores_for_query(iq: np.ndarray, ik_rows: np.ndarray, p: int,
                           score_type: str = "max") -> np.ndarray:
    """score[j] = the score_type reduction over tokens t of block j with t <= p
    of iq . ik[t] (max by default).

    ``ik_rows`` holds at least the sequence's tokens 0..p (float64).
    """
    nb = num_visible_blocks(p)
    if nb == 0:
        return np.zeros(0)
    dots = ik_rows[: p + 1] @ iq                      # [p+1]
    if score_type != "max":
        return np.array([reduce_block(dots[j * BLOCK:min((j + 1) * BLOCK, p + 1)], score_type,
                                      iq.shape[-1]) for j in range(nb)])
    pad = nb * BLOCK - (p + 1)
    dots = np.concatenate([dots, np.full(pad, -np.inf)])
    return dots.reshape(nb, BLOCK).max(axis=1)


def block_scores(inp: dict) -> np.ndarray:
    """Scores [T, Hidx, max_blocks] float64 of ``inp["score_type"]`` (max when
    absent); -inf for blocks past the query.

    The queries of one sequence and index head are scored together with one
    matrix product (chunks of 1024 queries); each row is then masked to its
    own position and reduced per block exactly as ``block_scores_for_query``.
    """
    iq_all = decode(inp["idx_q"], inp["idx_dtype"])
    T, Hidx, _ = iq_all.shape
    MB = inp["block_table"].shape[1]
    out = np.full((T, Hidx, MB), -np.inf)
    pos = query_positions(inp["seq_lens"], inp.get("cu_seqlens_q"), inp.get("positions"))
    by_seq = {}
    for t, (b, p) in enumerate(pos):
        by_seq.setdefault(b, []).append((t, p))
    for b, items in by_seq.items():
        L = int(inp["seq_lens"][b])
        if L <= 0:
            continue
        nbL = num_visible_blocks(L - 1)
        for h in range(Hidx):
            ik = decode(_gather_rows_raw(inp["idx_k_pool"], inp["block_table"][b], h, L),
                        inp["idx_dtype"])
            for c0 in range(0, len(items), 1024):
                chunk = items[c0:c0 + 1024]
                ts = np.array([t for t, _ in chunk])
                ps = np.array([p for _, p in chunk])
                dots = np.full((len(chunk), nbL * BLOCK), -np.inf)
                dots[:, :L] = iq_all[ts, h] @ ik.T
                tok = np.arange(nbL * BLOCK)
                vis = tok[None, :] <= ps[:, None]
                dots[~vis] = -np.inf
                d3 = dots.reshape(len(chunk), nbL, BLOCK)
                v3 = vis.reshape(len(chunk), nbL, BLOCK)
                st = inp.get("score_type", "max")
                if st == "max":
                    s = d3.max(axis=2)
                elif st == "mean":
                    cnt = v3.sum(axis=2)
                    s = np.where(v3, d3, 0.0).sum(axis=2) / np.maximum(cnt, 1)
                elif st == "lse":
                    z = d3 / math.sqrt(iq_all.shape[-1])
                    m = z.max(axis=2)
                    msafe = np.where(np.isfinite(m), m, 0.0)
                    with np.errstate(divide="ignore"):   # blocks past the query: log 0
                        s = msafe + np.log(np.where(v3, np.exp(z - msafe[..., None]), 0.0)
                                           .sum(axis=2))
                else:
                    raise ValueError(st)
                for r, (t, p) in enumerate(chunk):
                    nb = num_visible_blocks(p)
                    out[t, h, :nb] = s[r, :nb]
    return out


def _gather_rows_raw(pool: np.ndarray, bt_row: np.ndarray, head: int, n_tokens: int):
    """Raw stored rows 0..n_tokens-1 of one head of a sequence."""
    nbk = (n_tokens + BLOCK - 1) // BLOCK
    pages = np.asarray(bt_row[:nbk], dtype=np.int64)
    rows = pool[pages, head].reshape(nbk * BLOCK, pool.shape[-1])
    return rows[:n_tokens]


def _gather_values(pool: np.ndarray, bt_row: np.ndarray, head: int, n_tokens: int, dtype: str,
                   scale: float, D: int) -> np.ndarray:
    """Values (float64) of rows 0..n_tokens-1 of one head of a sequence."""
    if dtype in ("mxfp4", "mxfp6"):
        nbk = (n_tokens + BLOCK - 1) // BLOCK
        pages = np.asarray(bt_row[:nbk], dtype=np.int64)
        dec = mxfp4_decode_runs if dtype == "mxfp4" else mxfp6_decode_runs
        vals = dec(pool[pages, head], D, scale)
        return vals.reshape(nbk * BLOCK, D)[:n_tokens]
    return decode(_gather_rows_raw(pool, bt_row, head, n_tokens), dtype, scale)


# --------------------------------------------------------------------------
# Step 2: forced blocks and top-k selection
# --------------------------------------------------------------------------

def forced_blocks(nb: int, init: int, local: int) -> list:
    """Init blocks {0..init-1} and local blocks {nb-local..nb-1}, within [0,nb)."""
    f = set(range(min(init, nb)))
    f.update(range(max(0, nb - local), nb))
    return sorted(f)


def select_for_query(scores: np.ndarray, nb: int, topk: int, init: int, local: int,
                     forced_in_budget: bool = False) -> list:
    """S = forced blocks plus the top-k of the others by (score desc, index asc),
    returned in ascending block order.

    ``forced_in_budget`` is the other reading of the budget (the sglang page
    sizes its dense fallback over the selected blocks for topk_blocks *
    block_size_k tokens): the forced blocks count against topk, so only
    max(topk - |F|, 0) others join them."""
    forced = forced_blocks(nb, init, local)
    fset = set(forced)
    cand = [j for j in range(nb) if j not in fset]
    cand.sort(key=lambda j: (-float(scores[j]), j))
    k = max(topk - len(forced), 0) if forced_in_budget else topk
    chosen = cand[: min(k, len(cand))]
    return sorted(fset.union(chosen))


def kmax(topk: int, init: int, local: int) -> int:
    return topk + init + local


def select(inp: dict, scores: np.ndarray):
    """sel [T, Hidx, Kmax] int32 (-1 padded, ascending) and count [T, Hidx]."""
    T, Hidx, _ = scores.shape
    K = kmax(inp["topk"], inp["init"], inp["local"])
    sel = np.full((T, Hidx, K), -1, dtype=np.int32)
    cnt = np.zeros((T, Hidx), dtype=np.int32)
    pos = query_positions(inp["seq_lens"], inp.get("cu_seqlens_q"), inp.get("positions"))
    for t, (b, p) in enumerate(pos):
        nb = num_visible_blocks(p)
        for h in range(Hidx):
            s = select_for_query(scores[t, h], nb, inp["topk"], inp["init"], inp["local"],
                                 bool(inp.get("forced_in_budget", False)))
            sel[t, h, : len(s)] = s
            cnt[t, h] = len(s)
    return sel, cnt


# --------------------------------------------------------------------------
# Step 3: exact softmax attention restricted to the selected blocks
# --------------------------------------------------------------------------

def visible_rows(blocks, p: int) -> np.ndarray:
    """Token positions of the selected blocks that are <= p, ascending."""
    rows = []
    for j in sorted(blocks):
        lo = j * BLOCK
        hi = min(lo + BLOCK - 1, p)
        rows.extend(range(lo, hi + 1))
    return np.asarray(rows, dtype=np.int64)


def softmax_attention(qh: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      return_weights: bool = False):
    """out[h] = sum_t w[h,t] v[t], w = softmax_t(scale * q[h] . k[t]);
    lse[h] = log sum_t exp(scale * q[h] . k[t]).  qh [G,D], k/v [n,D]."""
    G = qh.shape[0]
    if k.shape[0] == 0:
        o = np.zeros((G, v.shape[1]))
        lse = np.full(G, -np.inf)
        return (o, lse, np.zeros((G, 0))) if return_weights else (o, lse)
    z = scale * (qh @ k.T)                            # [G, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    w = e / s
    o = w @ v
    lse = (m + np.log(s))[:, 0]
    return (o, lse, w) if return_weights else (o, lse)


def attend(inp: dict, sel: np.ndarray, cnt: np.ndarray, scale: Optional[float] = None):
    """out [T, Hq, D] and lse [T, Hq] for the given selection."""
    q_all = decode(inp["q"], inp["q_dtype"])
    T, Hq, D = q_all.shape
    Hkv, Hidx = inp["Hkv"], inp["Hidx"]
    G = Hq // Hkv
    gpi = Hkv // Hidx
    sc = (1.0 / math.sqrt(D)) if not scale else float(scale)
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    pos = query_positions(inp["seq_lens"], inp.get("cu_seqlens_q"), inp.get("positions"))
    by_seq = {}
    for t, (b, p) in enumerate(pos):
        by_seq.setdefault(b, []).append((t, p))
    for b, items in by_seq.items():
        L = int(inp["seq_lens"][b])
        if L <= 0:
            continue
        for g in range(Hkv):
            kr = _gather_values(inp["k_pool"], inp["block_table"][b], g, L, inp["kv_dtype"],
                                inp.get("k_scale", 1.0), D)
            vr = _gather_values(inp["v_pool"], inp["block_table"][b], g, L, inp["kv_dtype"],
                                inp.get("v_scale", 1.0), D)
            h = g // gpi
            for t, p in items:
                blocks = sel[t, h, : cnt[t, h]]
                rows = visible_rows(blocks, p)
                o, l = softmax_attention(q_all[t, g * G:(g + 1) * G], kr[rows], vr[rows], sc)
                out[t, g * G:(g + 1) * G] = o
                lse[t, g * G:(g + 1) * G] = l
    return out, lse


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge attention over disjoint key sets: lse = log sum_c exp(lse_c),
    out = sum_c exp(lse_c - lse) o_c.  o_parts [C, ..., D], lse_parts [C, ...]."""
    m = np.max(lse_parts, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe)
    s = w.sum(axis=0)
    lse = np.where(s > 0, m_safe + np.log(np.where(s > 0, s, 1.0)), -np.inf)
    wn = np.where(s > 0, w / np.where(s > 0, s, 1.0), 0.0)
    return (wn[..., None] * o_parts).sum(axis=0), lse


# --------------------------------------------------------------------------
# Whole path
# --------------------------------------------------------------------------

def sparse_attention(inp: dict, scale: Optional[float] = None) -> dict:
    """Score, select and attend for every query token (decode or prefill)."""
    scores = block_scores(inp)
    sel, cnt = select(inp, scores)
    out, lse = attend(inp, sel, cnt, scale)
    return dict(scores=scores, sel=sel, count=cnt, out=out, lse=lse)


# --------------------------------------------------------------------------
# Paged append of the new tokens (the step before the path)
# --------------------------------------------------------------------------
#
# The sglang page's backend stores the new tokens' K, V and index keys into
# its pool at ``out_cache_loc`` before it attends (the pool's
# ``set_fused_kv_index_buffer``; its body is not on the pages).  Reading
# taken here: ``out_cache_loc`` holds flat token slots of the paged pool, slot
# s living in page s // 128 at offset s % 128; slots outside the pool (e.g.
# -1 padding) are not written.  A bf16 or f32 pool stores the value as given;
# an fp8 pool stores the e4m3fn code of x / scale (per-tensor k_scale or
# v_scale, the vLLM page's fp8 cache scales), the division done in float32,
# clamped to +-448, rounded to nearest with ties to even.


def fp8_e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8).

    From the format definition alone: each value is clamped to +-448 (the
    largest finite magnitude), then takes the code of the same sign whose
    value is nearest, an exact tie going to the code with an even mantissa
    (its lowest bit clear); a negative value that rounds to zero keeps its
    sign (code 0x80).  NaN becomes the NaN code of its sign (0x7F / 0xFF).
    """
    return _encode_nearest(y, fp8_e4m3fn_table(), 0x7F, 0x7F)


def fp8_e5m2_encode(y: np.ndarray) -> np.ndarray:
    """float32 values -> e5m2 codes (uint8): the same rule as the e4m3
    encoder over the E5M2 codes: clamp to +-57344 (the largest finite
    magnitude, so the stored code saturates instead of becoming inf), nearest
    code of the same sign, ties to the even mantissa; NaN -> 0x7F / 0xFF."""
    return _encode_nearest(y, fp8_e5m2_table(), 0x7C, 0x7F)


def _encode_nearest(y, tab, n_finite: int, nan_code: int) -> np.ndarray:
    """Codes 0..n_finite-1 are the finite non-negative ones, ascending."""
    top = float(tab[n_finite - 1])
    y32 = np.asarray(y, dtype=np.float32)
    flat = y32.reshape(-1)
    neg = np.signbit(flat)
    mag = np.abs(flat.astype(np.float64))
    nan = np.isnan(mag)
    mag = np.minimum(np.where(nan, 0.0, mag), top)
    codes = np.arange(n_finite)              # finite non-negative codes
    vals = tab[codes]                        # ascending magnitudes
    dist = np.abs(mag[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best                      # one or two neighbouring codes
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    out = codes[pick].astype(np.uint8)
    out = np.where(nan, np.uint8(nan_code), out)
    out = np.where(neg, out | np.uint8(0x80), out).astype(np.uint8)
    return out.reshape(y32.shape)


def store_values(src: np.ndarray, src_dtype: str, pool_dtype: str, scale: float = 1.0):
    """New values in their source representation (bf16 bits, f32) -> the
    pool's stored representation."""
    if pool_dtype == src_dtype:
        return np.array(src, copy=True)
    if pool_dtype in ("fp8", "fp8_e5m2") and src_dtype == "bf16":
        x32 = decode(src, "bf16").astype(np.float32)   # exact
        y32 = x32 / np.float32(scale)                  # IEEE float32 division
        return fp8_e4m3fn_encode(y32) if pool_dtype == "fp8" else fp8_e5m2_encode(y32)
    raise ValueError((src_dtype, pool_dtype))


def append_kv(k_pool, v_pool, idx_k_pool, k_new, v_new, idx_k_new, slots, *,
              kv_src: str, kv_dtype: str, idx_dtype: str, k_scale: float = 1.0,
              v_scale: float = 1.0, idx_v_pool=None, idx_v_new=None):
    """Pools (stored arrays, [P, H, 128, D]) with token t's rows written at
    slot slots[t]; returns new arrays, the inputs are left unchanged.
    k_new / v_new [T, Hkv, D] and idx_k_new [T, Hidx, Di] are given in their
    source representation (kv_src: bf16 bits or f32; index keys already in
    idx_dtype).  With an index-value pool, idx_v_new [T, Hidx, Di] (idx_dtype)
    is stored beside the index keys and the new pool is returned fourth."""
    k_pool, v_pool, idx_k_pool = (np.array(a, copy=True) for a in (k_pool, v_pool, idx_k_pool))
    if idx_v_pool is not None:
        idx_v_pool = np.array(idx_v_pool, copy=True)
    P = k_pool.shape[0]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0 or s >= P * BLOCK:
            continue
        page, off = divmod(int(s), BLOCK)
        if kv_dtype == "mxfp4":
            for pool, new, sc in ((k_pool, k_new, k_scale), (v_pool, v_new, v_scale)):
                _store_mxfp4_row(pool, page, off, new[t], kv_src, sc)
        elif kv_dtype == "mxfp6":
            for pool, new, sc in ((k_pool, k_new, k_scale), (v_pool, v_new, v_scale)):
                _store_mxfp6_row(pool, page, off, new[t], kv_src, sc)
        else:
            k_pool[page, :, off, :] = store_values(k_new[t], kv_src, kv_dtype, k_scale)
            v_pool[page, :, off, :] = store_values(v_new[t], kv_src, kv_dtype, v_scale)
        idx_k_pool[page, :, off, :] = store_values(idx_k_new[t], idx_dtype, idx_dtype)
        if idx_v_pool is not None:
            idx_v_pool[page, :, off, :] = store_values(idx_v_new[t], idx_dtype, idx_dtype)
    if idx_v_pool is not None:
        return k_pool, v_pool, idx_k_pool, idx_v_pool
    return k_pool, v_pool, idx_k_pool


def _store_mxfp4_row(pool, page, off, new_row, src, scale):
    """One token's rows [H, D] (bf16 bits) into an MX-fp4 pool: the float32
    quotient x / scale encoded per group of 32 (mxfp4_encode_rows)."""
    x32 = decode(new_row, src).astype(np.float32) / np.float32(scale)
    codes, sc = mxfp4_encode_rows(x32)
    D = new_row.shape[-1]
    nc = BLOCK * D // 2
    pool[page, :, off * D // 2:(off + 1) * D // 2] = codes
    pool[page, :, nc + off * D // MXFP4_GROUP:nc + (off + 1) * D // MXFP4_GROUP] = sc


def _store_mxfp6_row(pool, page, off, new_row, src, scale):
    """One token's rows [H, D] (bf16 bits) into an MX-fp6 pool: the float32
    quotient x / scale encoded per group of 32 (mxfp6_encode_rows)."""
    x32 = decode(new_row, src).astype(np.float32) / np.float32(scale)
    codes, sc = mxfp6_encode_rows(x32)
    D = new_row.shape[-1]
    nc = BLOCK * D * 3 // 4
    pool[page, :, off * D * 3 // 4:(off + 1) * D * 3 // 4] = codes
    pool[page, :, nc + off * D // MXFP4_GROUP:nc + (off + 1) * D // MXFP4_GROUP] = sc


# --------------------------------------------------------------------------
# Index-value branch
# --------------------------------------------------------------------------
#
# The sglang page's backend keeps an index-value cache beside the index keys
# (set_fused_kv_index_buffer stores idx_v unless the layer is listed in
# disable_value_layer_ids), hands both caches to the sparse ops with
# disable_index_value, and gets back an index output idx_o of
# num_idx_heads * sparse_index_dim values per token next to the attention
# output.  What the ops compute is not on the pages.  Reading taken here: per
# index head, plain softmax attention of the index query over the index keys
# and index values of every token the query can see (t <= p, all blocks: the
# index branch already scores every block), with the usual scale
# 1/sqrt(idx_dim).


def index_value_attention(inp: dict, scale: Optional[float] = None):
    """idx_out [T, Hidx, Di] and its lse [T, Hidx] (natural log of the scaled
    logits); an index query with no visible token gives zeros and -inf."""
    iq_all = decode(inp["idx_q"], inp["idx_dtype"])
    T, Hidx, Di = iq_all.shape
    sc = (1.0 / math.sqrt(Di)) if not scale else float(scale)
    out = np.zeros((T, Hidx, Di))
    lse = np.full((T, Hidx), -np.inf)
    pos = query_positions(inp["seq_lens"], inp.get("cu_seqlens_q"), inp.get("positions"))
    for t, (b, p) in enumerate(pos):
        if p < 0:
            continue
        for h in range(Hidx):
            k = decode(_gather_rows_raw(inp["idx_k_pool"], inp["block_table"][b], h, p + 1),
                       inp["idx_dtype"])
            v = decode(_gather_rows_raw(inp["idx_v_pool"], inp["block_table"][b], h, p + 1),
                       inp["idx_dtype"])
            o, l = softmax_attention(iq_all[t, h][None, :], k, v, sc)
            out[t, h] = o[0]
            lse[t, h] = l[0]
    return out, lse


# --------------------------------------------------------------------------
# MX-fp4 K/V pools
# --------------------------------------------------------------------------
#
# The vLLM page keeps 4-bit K/V caches with per-block scales in per-head
# K/V slots (MiniMaxM3SparseMSANvfp4Backend).  The gfx950 counterpart taken
# here is the OCP Microscaling MXFP4 format: E2M1 element codes, a shared
# E8M0 scale per 32 consecutive elements.  Pool layout per (page, head): the
# 128 x D / 2 code bytes (two codes per byte, element 2i in the low nibble),
# then the 128 x D / 32 scale bytes; the per-tensor k_scale / v_scale
# multiply on top.

MXFP4_GROUP = 32


def fp4_e2m1_table() -> np.ndarray:
    """Values of the 16 OCP E2M1 codes: s.ee.m, exponent bias 1; exponent
    field 0 encodes the subnormal m * 0.5; no infinities or NaN."""
    tab = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        tab[code] = sign * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return tab


def e8m0_table() -> np.ndarray:
    """Values of the 256 E8M0 scale codes: 2^(code - 127); 0xFF is NaN."""
    tab = np.array([2.0 ** (c - 127) for c in range(256)], dtype=np.float64)
    tab[255] = math.nan
    return tab


def mxfp4_run_bytes(D: int) -> int:
    return BLOCK * D // 2 + BLOCK * D // MXFP4_GROUP


def mxfp4_decode_runs(runs: np.ndarray, D: int, scale: float = 1.0) -> np.ndarray:
    """[..., run bytes] uint8 -> [..., 128, D] float64 values times scale."""
    runs = np.asarray(runs, dtype=np.uint8)
    nc = BLOCK * D // 2
    codes = runs[..., :nc].reshape(runs.shape[:-1] + (BLOCK, D // 2))
    sc = runs[..., nc:].reshape(runs.shape[:-1] + (BLOCK, D // MXFP4_GROUP))
    tab = fp4_e2m1_table()
    el = np.empty(runs.shape[:-1] + (BLOCK, D), dtype=np.float64)
    el[..., 0::2] = tab[codes & 0xF]
    el[..., 1::2] = tab[codes >> 4]
    s = e8m0_table()[sc]
    return el * np.repeat(s, MXFP4_GROUP, axis=-1) * float(scale)


def fp4_e2m1_encode(y: np.ndarray) -> np.ndarray:
    """Magnitudes to E2M1 codes: nearest of the eight values, an exact tie to
    the even mantissa, clamped at 6; the sign is kept (-0 -> 0x8)."""
    y = np.asarray(y, dtype=np.float64)
    tab = fp4_e2m1_table()[:8]
    mag = np.minimum(np.abs(np.where(np.isnan(y), 0.0, y)), 6.0)
    dist = np.abs(mag[..., None] - tab)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    even = cand & ((np.arange(8) & 1) == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (pick | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def mxfp4_encode_rows(x32: np.ndarray):
    """Rows [..., D] of float32 values -> (codes [..., D / 2], scale codes
    [..., D / 32]) by the OCP rule: per group of 32, the shared exponent is
    floor(log2(max |x|)) - 2 (2 being E2M1's largest exponent), clamped to the
    E8M0 range (an all-zero group takes code 0), and every element is
    encoded as x / 2^exponent; a group holding a NaN gets the NaN scale code."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // MXFP4_GROUP, MXFP4_GROUP))
    nan = np.isnan(g).any(axis=-1)
    amax = np.max(np.abs(np.where(np.isnan(g), 0.0, g)), axis=-1)
    _, e = np.frexp(amax)                       # amax = f * 2^e, f in [0.5, 1)
    k = np.where(amax > 0, e - 1 - 2, -127)
    sc = np.clip(k + 127, 0, 254)
    X = np.ldexp(1.0, (sc - 127).astype(np.int64))
    codes = fp4_e2m1_encode(g / X[..., None]).reshape(x.shape)
    codes = np.where(np.repeat(nan, MXFP4_GROUP, axis=-1), np.uint8(0), codes)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, np.where(nan, 255, sc).astype(np.uint8)


def mxfp4_encode_run_rows(x32: np.ndarray):
    """Convenience: [..., 128, D] float32 -> [..., run bytes] (codes, then scales)."""
    codes, sc = mxfp4_encode_rows(x32)
    lead = codes.shape[:-2]
    return np.concatenate([codes.reshape(lead + (-1,)), sc.reshape(lead + (-1,))], axis=-1)


# --------------------------------------------------------------------------
# MX-fp6 K/V pools
# --------------------------------------------------------------------------
#
# The other microscaling width gfx950 converts in hardware, beside MX-fp4:
# OCP FP6 E2M3 element codes (s.ee.mmm, exponent bias 1; exponent field 0
# encodes the subnormal m / 8; the largest value 7.5; no infinities or NaN)
# with an E8M0 scale per 32 consecutive elements.  A group's 32 codes pack
# into 24 bytes, element i at bits 6 i .. 6 i + 5 of the group read as one
# little-endian number.  Pool layout per (page, head): the 128 x D x 3 / 4
# code bytes, then the 128 x D / 32 scale bytes; k_scale / v_scale multiply
# on top.

def fp6_e2m3_table() -> np.ndarray:
    """Values of the 64 E2M3 codes."""
    tab = np.empty(64, dtype=np.float64)
    for code in range(64):
        sign = -1.0 if code & 0x20 else 1.0
        e = (code >> 3) & 0x3
        m = code & 0x7
        tab[code] = sign * (m / 8.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 1))
    return tab


def mxfp6_run_bytes(D: int) -> int:
    return BLOCK * D * 3 // 4 + BLOCK * D // MXFP4_GROUP


def fp6_pack(codes: np.ndarray) -> np.ndarray:
    """[..., D] codes (0..63) -> [..., 3 D / 4] bytes: every four codes are
    three bytes, c0 | c1 << 6 | c2 << 12 | c3 << 18 little-endian."""
    c = np.asarray(codes, dtype=np.uint32).reshape(codes.shape[:-1] + (-1, 4))
    v = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
    b = np.stack([v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF], axis=-1)
    return b.reshape(codes.shape[:-1] + (-1,)).astype(np.uint8)


def fp6_unpack(packed: np.ndarray) -> np.ndarray:
    """Inverse of fp6_pack."""
    b = np.asarray(packed, dtype=np.uint32).reshape(packed.shape[:-1] + (-1, 3))
    v = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    c = np.stack([(v >> (6 * i)) & 0x3F for i in range(4)], axis=-1)
    return c.reshape(packed.shape[:-1] + (-1,)).astype(np.uint8)


def mxfp6_decode_runs(runs: np.ndarray, D: int, scale: float = 1.0) -> np.ndarray:
    """[..., run bytes] uint8 -> [..., 128, D] float64 values times scale."""
    runs = np.asarray(runs, dtype=np.uint8)
    nc = BLOCK * D * 3 // 4
    codes = fp6_unpack(runs[..., :nc].reshape(runs.shape[:-1] + (BLOCK, D * 3 // 4)))
    sc = runs[..., nc:].reshape(runs.shape[:-1] + (BLOCK, D // MXFP4_GROUP))
    el = fp6_e2m3_table()[codes]
    s = e8m0_table()[sc]
    return el * np.repeat(s, MXFP4_GROUP, axis=-1) * float(scale)


def fp6_e2m3_encode(y: np.ndarray) -> np.ndarray:
    """Magnitudes to E2M3 codes: nearest of the 32 values, an exact tie to the
    even mantissa, clamped at 7.5; the sign is kept (-0 -> 0x20)."""
    y = np.asarray(y, dtype=np.float64)
    tab = fp6_e2m3_table()[:32]
    mag = np.minimum(np.abs(np.where(np.isnan(y), 0.0, y)), 7.5)
    dist = np.abs(mag[..., None] - tab)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    even = cand & ((np.arange(32) & 1) == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (pick | np.where(np.signbit(y), 0x20, 0)).astype(np.uint8)


def mxfp6_encode_rows(x32: np.ndarray):
    """Rows [..., D] of float32 values -> (packed codes [..., 3 D / 4], scale
    codes [..., D / 32]) by the OCP rule: per group of 32, the shared exponent
    floor(log2(max |x|)) - 2 (2 being E2M3's largest exponent), clamped to the
    E8M0 range (an all-zero group takes code 0); every element encoded as
    x / 2^exponent; a group holding a NaN gets the NaN scale code and zero
    codes."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // MXFP4_GROUP, MXFP4_GROUP))
    nan = np.isnan(g).any(axis=-1)
    amax = np.max(np.abs(np.where(np.isnan(g), 0.0, g)), axis=-1)
    _, e = np.frexp(amax)
    k = np.where(amax > 0, e - 1 - 2, -127)
    sc = np.clip(k + 127, 0, 254)
    X = np.ldexp(1.0, (sc - 127).astype(np.int64))
    codes = fp6_e2m3_encode(g / X[..., None]).reshape(x.shape)
    codes = np.where(np.repeat(nan, MXFP4_GROUP, axis=-1), np.uint8(0), codes)
    return fp6_pack(codes), np.where(nan, 255, sc).astype(np.uint8)


def mxfp6_encode_run_rows(x32: np.ndarray):
    """Convenience: [..., 128, D] float32 -> [..., run bytes] (codes, then scales)."""
    codes, sc = mxfp6_encode_rows(x32)
    lead = codes.shape[:-2]
    return np.concatenate([codes.reshape(lead + (-1,)), sc.reshape(lead + (-1,))], axis=-1)
