"""Python entry points with the names of the C ABI (argument marshalling only).

Tensors are torch tensors on the GPU; each call passes their device pointers
and the current stream to libmsa.so, which does every step of the path in its
own kernels.  The only thing this layer does besides marshalling is allocate
the caller-side outputs and workspace with torch when they are not given.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (MSA_BF16, MSA_F32, MSA_FP8_E4M3, MSA_FP8_E5M2, MSA_MXFP4, MSA_MXFP6, Params,
                   check, load)

BLOCK = 128


# block score types by name, as msa_params_t.score_type codes them
SCORE_TYPES = {"max": 0, "mean": 1, "lse": 2}


@dataclass
class MsaConfig:
    """Model parameters (see msa_params_t in include/msa.h)."""

    num_q_heads: int
    num_kv_heads: int
    num_idx_heads: int
    head_dim: int = 128
    idx_dim: int = 128
    topk: int = 16
    init_blocks: int = 1
    local_blocks: int = 2
    softmax_scale: float = 0.0
    q_dtype: str = "bf16"
    kv_dtype: str = "bf16"
    idx_dtype: str = "bf16"
    k_scale: float = 1.0
    v_scale: float = 1.0
    block_size: int = BLOCK
    forced_in_budget: bool = False  # forced blocks count inside topk
    index_value: bool = False       # the index-value branch (idx_v pool, idx_out)
    score_type: str = "max"         # block score: "max", "mean" or "lse"

    @property
    def kmax(self) -> int:
        return self.topk + self.init_blocks + self.local_blocks

    def params(self) -> Params:
        code = {"bf16": MSA_BF16, "f32": MSA_F32, "fp8": MSA_FP8_E4M3,
                "fp8_e5m2": MSA_FP8_E5M2, "mxfp4": MSA_MXFP4, "mxfp6": MSA_MXFP6}
        return Params(self.num_q_heads, self.num_kv_heads, self.num_idx_heads, self.head_dim,
                      self.idx_dim, self.block_size, self.topk, self.init_blocks,
                      self.local_blocks, self.softmax_scale, code[self.q_dtype],
                      code[self.kv_dtype], code[self.idx_dtype], self.k_scale, self.v_scale,
                      int(self.forced_in_budget), int(self.index_value),
                      SCORE_TYPES[self.score_type])

    @staticmethod
    def from_spec(spec: dict) -> "MsaConfig":
        return MsaConfig(num_q_heads=spec["Hq"], num_kv_heads=spec["Hkv"],
                         num_idx_heads=spec["Hidx"], head_dim=spec["D"], idx_dim=spec["Di"],
                         topk=spec["topk"], init_blocks=spec["init"],
                         local_blocks=spec["local"], q_dtype=spec.get("q", "bf16"),
                         kv_dtype=spec.get("kv", "bf16"), idx_dtype=spec.get("idx", "bf16"),
                         k_scale=float(spec.get("k_scale", 1.0)),
                         v_scale=float(spec.get("v_scale", 1.0)),
                         forced_in_budget=bool(spec.get("forced_in_budget", False)),
                         index_value=bool(spec.get("idx_value", False)),
                         score_type=spec.get("score_type", "max"))


def blocks_from_tokens(init_tokens: int, local_tokens: int, block_size: int = BLOCK):
    """Block counts for token-denominated settings, as the sglang backend derives
    them: init = ceil(init_tokens / bs); local = ceil(local_tokens / bs) + 1 (the
    extra block is the query's own, partially filled one)."""
    init = (init_tokens + block_size - 1) // block_size
    local = (local_tokens + block_size - 1) // block_size + 1
    return init, local


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_i32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.int32:
            raise ValueError("index tensors must be int32")


def version() -> int:
    return int(load().msa_version())


def decode_workspace_size(cfg: MsaConfig, num_seqs: int, max_blocks: int) -> int:
    p = cfg.params()
    n = load().msa_decode_workspace_size(ctypes.byref(p), num_seqs, max_blocks)
    if n == 0:
        check(_lib.MSA_ERR_INVALID_ARG if num_seqs >= 0 else _lib.MSA_ERR_INVALID_ARG)
    return int(n)


def prefill_workspace_size(cfg: MsaConfig, num_seqs: int, num_q_tokens: int,
                           max_blocks: int) -> int:
    p = cfg.params()
    n = load().msa_prefill_workspace_size(ctypes.byref(p), num_seqs, num_q_tokens, max_blocks)
    if n == 0:
        check(_lib.MSA_ERR_UNSUPPORTED)
    return int(n)


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def block_score(cfg: MsaConfig, idx_q, idx_k_pool, block_table, seq_lens,
                cu_seqlens_q=None, scores=None, stream=None) -> torch.Tensor:
    """Step 1: scores [T, Hidx, max_blocks] (float32)."""
    _check_i32(block_table, seq_lens, cu_seqlens_q)
    B, MB = block_table.shape
    T = idx_q.shape[0]
    if scores is None:
        scores = torch.empty((T, cfg.num_idx_heads, MB), dtype=torch.float32,
                             device=idx_q.device)
    p = cfg.params()
    check(load().msa_block_score(ctypes.byref(p), _ptr(idx_q), _ptr(idx_k_pool),
                                 idx_k_pool.shape[0], _ptr(block_table), MB, _ptr(seq_lens),
                                 _ptr(cu_seqlens_q), B, T, _ptr(scores), _stream(stream)))
    return scores


def select_blocks(cfg: MsaConfig, scores, seq_lens, cu_seqlens_q=None, sel_blocks=None,
                  sel_count=None, stream=None):
    """Step 2: (sel_blocks [T, Hidx, Kmax], sel_count [T, Hidx]) int32."""
    _check_i32(seq_lens, cu_seqlens_q)
    T, Hidx, MB = scores.shape
    B = seq_lens.shape[0]
    dev = scores.device
    if sel_blocks is None:
        sel_blocks = torch.empty((T, Hidx, cfg.kmax), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((T, Hidx), dtype=torch.int32, device=dev)
    p = cfg.params()
    check(load().msa_select_blocks(ctypes.byref(p), _ptr(scores), MB, _ptr(seq_lens),
                                   _ptr(cu_seqlens_q), B, T, _ptr(sel_blocks),
                                   _ptr(sel_count), _stream(stream)))
    return sel_blocks, sel_count


def _idx_out(cfg: MsaConfig, q, idx_q, idx_out):
    if not cfg.index_value:
        return None
    if idx_out is None:
        idx_out = torch.empty((idx_q.shape[0], cfg.num_idx_heads, cfg.idx_dim), dtype=q.dtype,
                              device=q.device)
    return idx_out


def sparse_decode(cfg: MsaConfig, q, idx_q, k_pool, v_pool, idx_k_pool, block_table,
                  seq_lens, out=None, lse=None, sel_blocks=None, sel_count=None,
                  workspace=None, return_selection=False, stream=None, idx_v_pool=None,
                  idx_out=None):
    """Steps 1-3 for decode (one query per sequence).  Returns out [B, Hq, D]
    (and lse [B, Hq], sel_blocks, sel_count when asked for); with
    cfg.index_value, idx_out [B, Hidx, Di] (the index-value branch over
    idx_v_pool) comes last."""
    _check_i32(block_table, seq_lens)
    B, MB = block_table.shape
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    idx_out = _idx_out(cfg, q, idx_q, idx_out)
    if return_selection:
        if lse is None:
            lse = torch.empty((B, cfg.num_q_heads), dtype=torch.float32, device=dev)
        if sel_blocks is None:
            sel_blocks = torch.empty((B, cfg.num_idx_heads, cfg.kmax), dtype=torch.int32,
                                     device=dev)
        if sel_count is None:
            sel_count = torch.empty((B, cfg.num_idx_heads), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(decode_workspace_size(cfg, B, MB), dev)
    p = cfg.params()
    check(load().msa_sparse_decode(
        ctypes.byref(p), _ptr(q), _ptr(idx_q), _ptr(k_pool), _ptr(v_pool), _ptr(idx_k_pool),
        _ptr(idx_v_pool), k_pool.shape[0], _ptr(block_table), MB, _ptr(seq_lens), B, _ptr(out),
        _ptr(idx_out), _ptr(lse), _ptr(sel_blocks), _ptr(sel_count), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    res = (out, lse, sel_blocks, sel_count) if return_selection else (out,)
    if cfg.index_value:
        res = res + (idx_out,)
    return res if len(res) > 1 else res[0]


def sparse_decode_noalloc(cfg: MsaConfig, q, idx_q, k_pool, v_pool, idx_k_pool, block_table,
                          seq_lens, out, lse=None, sel_blocks=None, sel_count=None,
                          stream=None, idx_v_pool=None, idx_out=None):
    """msa_sparse_decode_noalloc: decode into the caller's ``out`` (and the
    optional lse / selection outputs) with the library's own per-GPU scratch
    as the workspace; nothing is allocated, here or in the library."""
    _check_i32(block_table, seq_lens)
    B, MB = block_table.shape
    p = cfg.params()
    check(load().msa_sparse_decode_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(idx_q), _ptr(k_pool), _ptr(v_pool), _ptr(idx_k_pool),
        _ptr(idx_v_pool), k_pool.shape[0], _ptr(block_table), MB, _ptr(seq_lens), B, _ptr(out),
        _ptr(idx_out), _ptr(lse), _ptr(sel_blocks), _ptr(sel_count), _stream(stream)))
    return out


def sparse_attend(cfg: MsaConfig, q, k_pool, v_pool, block_table, seq_lens, sel_blocks,
                  sel_count, out=None, lse=None, workspace=None, stream=None):
    """Step 3 alone (decode) over a given selection.  Returns (out, lse)."""
    _check_i32(block_table, seq_lens, sel_blocks, sel_count)
    B, MB = block_table.shape
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, cfg.num_q_heads), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(decode_workspace_size(cfg, B, MB), dev)
    p = cfg.params()
    check(load().msa_sparse_attend(
        ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
        _ptr(block_table), MB, _ptr(seq_lens), B, _ptr(sel_blocks), _ptr(sel_count),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def sparse_prefill(cfg: MsaConfig, q, idx_q, k_pool, v_pool, idx_k_pool, block_table,
                   seq_lens, cu_seqlens_q, out=None, lse=None, sel_blocks=None,
                   sel_count=None, workspace=None, return_selection=False, stream=None,
                   idx_v_pool=None, idx_out=None):
    """Steps 1-3 for chunked prefill (query tokens laid out by cu_seqlens_q);
    with cfg.index_value, idx_out [T, Hidx, Di] comes last."""
    _check_i32(block_table, seq_lens, cu_seqlens_q)
    B, MB = block_table.shape
    T = q.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    idx_out = _idx_out(cfg, q, idx_q, idx_out)
    if return_selection:
        if lse is None:
            lse = torch.empty((T, cfg.num_q_heads), dtype=torch.float32, device=dev)
        if sel_blocks is None:
            sel_blocks = torch.empty((T, cfg.num_idx_heads, cfg.kmax), dtype=torch.int32,
                                     device=dev)
        if sel_count is None:
            sel_count = torch.empty((T, cfg.num_idx_heads), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(prefill_workspace_size(cfg, B, T, MB), dev)
    p = cfg.params()
    check(load().msa_sparse_prefill(
        ctypes.byref(p), _ptr(q), _ptr(idx_q), _ptr(k_pool), _ptr(v_pool), _ptr(idx_k_pool),
        _ptr(idx_v_pool), k_pool.shape[0], _ptr(block_table), MB, _ptr(seq_lens),
        _ptr(cu_seqlens_q), B, T, _ptr(out), _ptr(idx_out), _ptr(lse), _ptr(sel_blocks),
        _ptr(sel_count), _ptr(workspace), workspace.numel(), _stream(stream)))
    res = (out, lse, sel_blocks, sel_count) if return_selection else (out,)
    if cfg.index_value:
        res = res + (idx_out,)
    return res if len(res) > 1 else res[0]


def append_kv(cfg: MsaConfig, k_new, v_new, idx_k_new, slot_mapping, k_pool, v_pool,
              idx_k_pool, stream=None, idx_v_new=None, idx_v_pool=None):
    """Write token t's K, V (k_new, v_new [T, Hkv, D]) and index keys
    (idx_k_new [T, Hidx, Di]) into the pools at slot slot_mapping[t] (int64;
    page s // 128, offset s % 128; slots outside the pool are skipped), in
    place.  fp8 pools (uint8) receive the e4m3 codes of x / k_scale (v_scale)."""
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    T = slot_mapping.shape[0]
    for t, rows in ((k_new, cfg.num_kv_heads), (v_new, cfg.num_kv_heads),
                    (idx_k_new, cfg.num_idx_heads)):
        if t.shape[0] != T or t.shape[1] != rows:
            raise ValueError("new rows must be [T, heads, dim] with T = len(slot_mapping)")
    p = cfg.params()
    check(load().msa_append_kv(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(idx_k_new),
                               _ptr(idx_v_new), _ptr(slot_mapping), T, _ptr(k_pool),
                               _ptr(v_pool), _ptr(idx_k_pool), _ptr(idx_v_pool),
                               k_pool.shape[0], _stream(stream)))


def fp8_dequant(codes: torch.Tensor, scale: float = 1.0, out=None, fmt: str = "fp8",
                stream=None):
    """fp8 codes (uint8; fmt "fp8" = e4m3, "fp8_e5m2") -> float32 values times
    scale, as the loaders do it.  fmt "mxfp4": ``codes`` holds n / 2 code bytes
    then n / 32 scale bytes (17 n / 32 bytes), and n values come back; fmt
    "mxfp6": 3 n / 4 code bytes then n / 32 scale bytes (25 n / 32 bytes)."""
    if codes.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2):
        raise ValueError("codes must be uint8, float8_e4m3fn or float8_e5m2")
    code = {"fp8": MSA_FP8_E4M3, "fp8_e5m2": MSA_FP8_E5M2, "mxfp4": MSA_MXFP4,
            "mxfp6": MSA_MXFP6}[fmt]
    per32 = {"mxfp4": 17, "mxfp6": 25}.get(fmt)
    n = codes.numel() if per32 is None else codes.numel() * 32 // per32
    if out is None:
        shape = codes.shape if per32 is None else (n,)
        out = torch.empty(shape, dtype=torch.float32, device=codes.device)
    if out.numel() < n:
        raise ValueError("out holds fewer values than the codes")
    check(load().msa_fp8_dequant(_ptr(codes), _ptr(out), n, float(scale), code,
                                 _stream(stream)))
    return out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
