"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching the GPU (runs without a GPU)."""

import ctypes
import os
import re

import pytest

import block_sparse_attention_score_amd as msa
from block_sparse_attention_score_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

FAKE = ctypes.c_void_p(0x10000)          # never dereferenced: validation fails first
FAKE_WS_MISALIGNED = ctypes.c_void_p(0x10010)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for need in ("msa_block_score", "msa_select_blocks", "msa_sparse_decode",
                 "msa_sparse_attend", "msa_sparse_prefill", "msa_decode_workspace_size",
                 "msa_prefill_workspace_size", "msa_fp8_e4m3_dequant", "msa_fp8_dequant",
                 "msa_append_kv",
                 "msa_status_string",
                 "msa_last_error", "msa_version"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = msa.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_params_struct_layout_matches_header():
    # 18 four-byte int32 / float fields, no padding
    assert ctypes.sizeof(_lib.Params) == 18 * 4


def base_cfg(**kw):
    c = dict(num_q_heads=16, num_kv_heads=2, num_idx_heads=2, head_dim=128, idx_dim=128,
             topk=16, init_blocks=1, local_blocks=2)
    c.update(kw)
    return msa.MsaConfig(**c)


def decode_call(cfg, num_seqs=4, max_blocks=16, ws=FAKE, ws_bytes=1 << 30, q=FAKE,
                num_pages=64):
    p = cfg.params()
    return msa.load().msa_sparse_decode(
        ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, None, num_pages, FAKE, max_blocks, FAKE,
        num_seqs, FAKE, None, None, None, None, ws, ws_bytes, None)


BAD_PARAMS = [
    (dict(topk=5), _lib.MSA_ERR_UNSUPPORTED),
    (dict(topk=64), _lib.MSA_ERR_UNSUPPORTED),
    (dict(head_dim=64), _lib.MSA_ERR_UNSUPPORTED),
    (dict(idx_dim=96), _lib.MSA_ERR_UNSUPPORTED),
    (dict(block_size=64), _lib.MSA_ERR_UNSUPPORTED),
    (dict(num_q_heads=15), _lib.MSA_ERR_INVALID_ARG),
    (dict(num_q_heads=48, num_kv_heads=2), _lib.MSA_ERR_UNSUPPORTED),   # G = 24
    (dict(num_idx_heads=3, num_kv_heads=2), _lib.MSA_ERR_UNSUPPORTED),
    (dict(num_kv_heads=0), _lib.MSA_ERR_INVALID_ARG),
    (dict(init_blocks=-1), _lib.MSA_ERR_INVALID_ARG),
    (dict(local_blocks=65), _lib.MSA_ERR_UNSUPPORTED),
    (dict(softmax_scale=float("nan")), _lib.MSA_ERR_INVALID_ARG),
    (dict(forced_in_budget=2), _lib.MSA_ERR_INVALID_ARG),
    (dict(q_dtype="fp8", kv_dtype="fp8"), _lib.MSA_ERR_UNSUPPORTED),
    (dict(q_dtype="f32", kv_dtype="bf16"), _lib.MSA_ERR_UNSUPPORTED),
    (dict(idx_dtype="fp8"), _lib.MSA_ERR_UNSUPPORTED),
    (dict(kv_dtype="fp8", k_scale=0.0), _lib.MSA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,code", BAD_PARAMS, ids=[str(k) for k, _ in BAD_PARAMS])
def test_bad_params_rejected(kw, code):
    assert decode_call(base_cfg(**kw)) == code
    assert msa.load().msa_last_error().decode()
    p = base_cfg(**kw).params()
    assert msa.load().msa_decode_workspace_size(ctypes.byref(p), 4, 16) == 0


@pytest.mark.parametrize("code", [-1, 3])
def test_bad_score_type_rejected(code):
    lib = msa.load()
    p = base_cfg().params()
    p.score_type = code
    assert lib.msa_decode_workspace_size(ctypes.byref(p), 4, 16) == 0
    assert "score_type" in lib.msa_last_error().decode()
    for name in ("mean", "lse"):
        p = base_cfg(score_type=name).params()
        assert p.score_type == msa.api.SCORE_TYPES[name]
        assert lib.msa_decode_workspace_size(ctypes.byref(p), 4, 16) > 0


def test_null_params_and_pointers():
    lib = msa.load()
    assert lib.msa_sparse_decode(None, *([FAKE] * 5), None, 64, FAKE, 16, FAKE, 4, FAKE, None,
                                 None, None, None, FAKE, 1 << 20, None) == _lib.MSA_ERR_INVALID_ARG
    assert decode_call(base_cfg(), q=None) == _lib.MSA_ERR_INVALID_ARG
    assert "NULL" in lib.msa_last_error().decode()


def test_shape_checks():
    assert decode_call(base_cfg(), max_blocks=0) == _lib.MSA_ERR_INVALID_ARG
    assert decode_call(base_cfg(), max_blocks=8193) == _lib.MSA_ERR_UNSUPPORTED
    assert decode_call(base_cfg(), num_seqs=-1) == _lib.MSA_ERR_INVALID_ARG
    assert decode_call(base_cfg(), num_pages=0) == _lib.MSA_ERR_INVALID_ARG


def test_workspace_checks():
    cfg = base_cfg()
    need = msa.decode_workspace_size(cfg, 4, 16)
    assert need > 0
    assert decode_call(cfg, ws=None) == _lib.MSA_ERR_WORKSPACE
    assert decode_call(cfg, ws_bytes=need - 1) == _lib.MSA_ERR_WORKSPACE
    assert decode_call(cfg, ws=FAKE_WS_MISALIGNED) == _lib.MSA_ERR_WORKSPACE


def test_workspace_size_grows_with_shape():
    cfg = base_cfg()
    a = msa.decode_workspace_size(cfg, 32, 256)
    b = msa.decode_workspace_size(cfg, 64, 256)
    c = msa.decode_workspace_size(cfg, 32, 1024)
    assert 0 < a < b and a < c
    # scores alone need B * Hidx * MB floats
    assert a >= 32 * 2 * 256 * 4


def test_selection_pairing_required():
    cfg = base_cfg()
    p = cfg.params()
    st = msa.load().msa_sparse_decode(
        ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, FAKE, 16, FAKE, 4, FAKE, None,
        None, FAKE, None, FAKE, 1 << 30, None)
    assert st == _lib.MSA_ERR_INVALID_ARG


def test_status_strings():
    lib = msa.load()
    for code in range(5):
        assert lib.msa_status_string(code)
    assert lib.msa_status_string(99) == b"unknown status"


def test_block_token_conversion_follows_backend_rule():
    # sglang backend: init = ceil(tokens / bs); local = ceil(tokens / bs) + 1
    assert msa.blocks_from_tokens(1, 1) == (1, 2)
    assert msa.blocks_from_tokens(128, 256) == (1, 3)
    assert msa.blocks_from_tokens(0, 0) == (0, 1)
    assert msa.blocks_from_tokens(129, 129) == (2, 3)


def test_prefill_workspace_and_token_limit():
    cfg = base_cfg()
    p = cfg.params()
    lib = msa.load()
    # key-major prefill (bf16 q): scores, selection, k2q lists and bf16 partials
    T, B, MB = 4096, 2, 64
    need = lib.msa_prefill_workspace_size(ctypes.byref(p), B, T, MB)
    kmax = cfg.topk + cfg.init_blocks + cfg.local_blocks
    G = cfg.num_q_heads // cfg.num_kv_heads
    partials = T * cfg.num_kv_heads * kmax * G * cfg.head_dim * 2
    assert need >= T * cfg.num_idx_heads * MB * 4 + partials
    # list entries pack the token index above an 8-bit slot
    assert lib.msa_prefill_workspace_size(ctypes.byref(p), B, (1 << 23) - 1, MB) > 0
    assert lib.msa_prefill_workspace_size(ctypes.byref(p), B, 1 << 23, MB) == 0
    assert "num_q_tokens" in lib.msa_last_error().decode()


def append_call(cfg, num_tokens=8, num_pages=16, **ptrs):
    p = cfg.params()
    args = dict(k_new=FAKE, v_new=FAKE, idx_k_new=FAKE, slots=FAKE, k_pool=FAKE, v_pool=FAKE,
                idx_k_pool=FAKE, idx_v_new=None, idx_v_pool=None)
    args.update(ptrs)
    return msa.load().msa_append_kv(ctypes.byref(p), args["k_new"], args["v_new"],
                                    args["idx_k_new"], args["idx_v_new"], args["slots"],
                                    num_tokens, args["k_pool"], args["v_pool"],
                                    args["idx_k_pool"], args["idx_v_pool"], num_pages, None)


def test_append_validation_before_launch():
    """msa_append_kv rejects bad arguments before it enqueues anything (the
    fake pointers are never dereferenced)."""
    lib = msa.load()
    for name in ("k_new", "v_new", "idx_k_new", "slots", "k_pool", "v_pool", "idx_k_pool"):
        assert append_call(base_cfg(), **{name: None}) == _lib.MSA_ERR_INVALID_ARG, name
        assert "NULL" in lib.msa_last_error().decode()
    assert append_call(base_cfg(), num_tokens=-1) == _lib.MSA_ERR_INVALID_ARG
    assert append_call(base_cfg(), num_pages=0) == _lib.MSA_ERR_INVALID_ARG
    assert append_call(base_cfg(kv_dtype="fp8", k_scale=0.0)) == _lib.MSA_ERR_INVALID_ARG
    assert append_call(base_cfg(kv_dtype="fp8_e5m2", v_scale=float("inf"))) == \
        _lib.MSA_ERR_INVALID_ARG
    assert append_call(base_cfg(q_dtype="f32", kv_dtype="fp8_e5m2")) == _lib.MSA_ERR_UNSUPPORTED
    # nothing to do: success without touching memory
    assert append_call(base_cfg(), num_tokens=0) == _lib.MSA_OK


def test_prefill_workspace_follows_the_chunk_path():
    """Short chunks (T <= 8 B) keep per-token split-K partials, long chunks the
    key-major lists and bf16 partials; the size is a function of the shapes."""
    cfg = base_cfg()
    lib = msa.load()
    p = cfg.params()
    short = lib.msa_prefill_workspace_size(ctypes.byref(p), 32, 8 * 32, 256)
    long_ = lib.msa_prefill_workspace_size(ctypes.byref(p), 32, 8 * 32 + 1, 256)
    assert short > 0 and long_ > 0 and long_ != short
    assert lib.msa_prefill_workspace_size(ctypes.byref(p), 32, 8 * 32, 256) == short


def test_msa_log_prints_the_launch_configuration():
    """MSA_LOG=1 makes every call print its launch configuration on stderr
    (read once per process, so this runs in a child process; the calls below
    have nothing to launch)."""
    import subprocess
    import sys
    code = (
        "import ctypes, block_sparse_attention_score_amd as msa\n"
        "from block_sparse_attention_score_amd import _lib\n"
        "cfg = msa.MsaConfig(num_q_heads=16, num_kv_heads=2, num_idx_heads=2)\n"
        "p = cfg.params(); F = ctypes.c_void_p(1 << 20)\n"
        "lib = msa.load()\n"
        "assert lib.msa_append_kv(ctypes.byref(p), F, F, F, None, F, 0, F, F, F, None, 16,"
        " None) == 0\n"
        "assert lib.msa_sparse_decode(ctypes.byref(p), F, F, F, F, F, None, 64, F, 16, F, 0, F,"
        " None, None, None, None, ctypes.c_void_p(1 << 20), 1 << 20, None) == 0\n")
    env = dict(os.environ, MSA_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120, cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    assert "[msa] msa_append_kv: T=0" in r.stderr
    assert "[msa] msa_sparse_decode: B=0" in r.stderr


def test_select_without_sequences_enqueues_nothing():
    """Token rows with no sequence to own them: nothing to select, and no
    kernel reads the one-entry offsets (the fake pointers are never used)."""
    p = base_cfg().params()
    lib = msa.load()
    assert lib.msa_select_blocks(ctypes.byref(p), FAKE, 16, FAKE, FAKE, 0, 5, FAKE, FAKE,
                                 None) == _lib.MSA_OK


def test_launch_sizes_past_the_grid_range_are_refused():
    """A launch whose grid would exceed a dispatch's 32-bit work-item count is
    refused on the host before anything is enqueued (fake pointers, never
    dereferenced): the decode attention grid (512 threads per workgroup), the
    append grid and the fp8 dequantisation grid."""
    lib = msa.load()
    # 5M sequences x 2 kv heads x 1 split = 10M attention workgroups
    assert decode_call(base_cfg(), num_seqs=5_000_000, max_blocks=8) == _lib.MSA_ERR_UNSUPPORTED
    assert "32-bit" in lib.msa_last_error().decode()
    p = base_cfg().params()
    assert lib.msa_sparse_attend(ctypes.byref(p), FAKE, FAKE, FAKE, 64, FAKE, 8, FAKE,
                                 5_000_000, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                 None) == _lib.MSA_ERR_UNSUPPORTED
    # 50M tokens x 96 sixteen-byte pieces each
    assert append_call(base_cfg(), num_tokens=50_000_000) == _lib.MSA_ERR_UNSUPPORTED
    assert lib.msa_fp8_dequant(FAKE, FAKE, 1 << 36, 1.0, _lib.MSA_FP8_E4M3,
                               None) == _lib.MSA_ERR_UNSUPPORTED
    # a long prefill chunk over more sequences than the list kernels' grid rows
    assert lib.msa_sparse_prefill(ctypes.byref(p), *([FAKE] * 5), None, 64, FAKE, 8, FAKE, FAKE,
                                  70000, 600000, FAKE, None, None, None, None, FAKE, 1 << 40,
                                  None) == _lib.MSA_ERR_UNSUPPORTED


def noalloc_call(cfg, num_seqs=4, max_blocks=16, q=FAKE):
    p = cfg.params()
    return msa.load().msa_sparse_decode_noalloc(
        ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, None, 64, FAKE, max_blocks, FAKE, num_seqs,
        FAKE, None, None, None, None, None)


def test_noalloc_decode_validates_before_touching_the_device():
    """The no-allocation decode checks its arguments and its scratch limit
    (16 MiB) on the host first; none of these calls reaches HIP."""
    lib = msa.load()
    assert noalloc_call(base_cfg(topk=5)) == _lib.MSA_ERR_UNSUPPORTED
    assert noalloc_call(base_cfg(), q=None) == _lib.MSA_ERR_INVALID_ARG
    assert noalloc_call(base_cfg(), max_blocks=0) == _lib.MSA_ERR_INVALID_ARG
    # 4096 sequences x 2 index heads x 8192 blocks of scores alone = 256 MiB
    need = msa.decode_workspace_size(base_cfg(), 4096, 8192)
    assert need > 16 << 20
    assert noalloc_call(base_cfg(), num_seqs=4096, max_blocks=8192) == _lib.MSA_ERR_UNSUPPORTED
    err = lib.msa_last_error().decode()
    assert "scratch" in err and str(need) in err


def test_index_value_pointers_follow_the_flag():
    """idx_v_pool / idx_out (idx_v_new / idx_v_pool for the append) are given
    exactly when params.index_value is set; checked before any launch."""
    lib = msa.load()
    on = base_cfg(index_value=True).params()
    off = base_cfg().params()
    args = lambda p, iv, io: (ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, iv, 64, FAKE, 16,
                              FAKE, 4, FAKE, io, None, None, None, FAKE, 1 << 30, None)
    assert lib.msa_sparse_decode(*args(on, None, None)) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_decode(*args(on, FAKE, None)) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_decode(*args(off, FAKE, FAKE)) == _lib.MSA_ERR_INVALID_ARG
    assert "index_value" in lib.msa_last_error().decode()
    assert append_call(base_cfg(index_value=True)) == _lib.MSA_ERR_INVALID_ARG
    assert append_call(base_cfg(), idx_v_new=FAKE, idx_v_pool=FAKE) == _lib.MSA_ERR_INVALID_ARG
    # the decode workspace holds the scores and the scan's value partials
    b = msa.decode_workspace_size(base_cfg(index_value=True), 8, 256)
    assert b >= 8 * 2 * 256 * 4 + 8 * 2 * 32 * 130 * 4
    bad = base_cfg().params()
    bad.index_value = 2
    assert lib.msa_decode_workspace_size(ctypes.byref(bad), 4, 16) == 0
