"""ctypes declarations of libmsa.so (the C ABI in include/msa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(5)
MSA_BF16, MSA_F32, MSA_FP8_E4M3, MSA_FP8_E5M2, MSA_MXFP4, MSA_MXFP6 = range(6)

STATUS_NAMES = {
    MSA_OK: "MSA_OK", MSA_ERR_INVALID_ARG: "MSA_ERR_INVALID_ARG",
    MSA_ERR_UNSUPPORTED: "MSA_ERR_UNSUPPORTED", MSA_ERR_WORKSPACE: "MSA_ERR_WORKSPACE",
    MSA_ERR_HIP: "MSA_ERR_HIP",
}


class Params(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_idx_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("init_blocks", ctypes.c_int32),
        ("local_blocks", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("idx_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("forced_in_budget", ctypes.c_int32),
        ("index_value", ctypes.c_int32),
        ("score_type", ctypes.c_int32),
    ]


class MsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_PP = ctypes.POINTER(Params)

# name -> (restype, argtypes)
SIGNATURES = {
    "msa_version": (_I32, []),
    "msa_status_string": (ctypes.c_char_p, [_I32]),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_decode_workspace_size": (_SZ, [_PP, _I32, _I32]),
    "msa_prefill_workspace_size": (_SZ, [_PP, _I32, _I32, _I32]),
    "msa_block_score": (_I32, [_PP, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _P, _P]),
    "msa_select_blocks": (_I32, [_PP, _P, _I32, _P, _P, _I32, _I32, _P, _P, _P]),
    "msa_sparse_decode": (_I32, [_PP, _P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _P,
                                 _P, _P, _P, _P, _P, _SZ, _P]),
    "msa_sparse_decode_noalloc": (_I32, [_PP, _P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                         _P, _P, _P, _P, _P, _P]),
    "msa_sparse_attend": (_I32, [_PP, _P, _P, _P, _I64, _P, _I32, _P, _I32, _P, _P, _P, _P,
                                 _P, _SZ, _P]),
    "msa_sparse_prefill": (_I32, [_PP, _P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32,
                                  _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "msa_append_kv": (_I32, [_PP, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _I64, _P]),
    "msa_fp8_e4m3_dequant": (_I32, [_P, _P, _I64, _F, _P]),
    "msa_fp8_dequant": (_I32, [_P, _P, _I64, _F, _I32, _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libmsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_attention_score_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != MSA_OK:
        detail = load().msa_last_error().decode(errors="replace")
        raise MsaError(status, detail)
