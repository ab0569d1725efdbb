"""GPU parity of the mean and log-sum-exp block scores (msa_params_t
score_type 1 and 2) against the fp64 oracle, through the C ABI: the decode
index scan (alone, and fused with the index-value branch), the prefill causal
GEMM scoring of long chunks and the page scan of short chunks, each followed
by the selection and the attention over it.

Scores follow the same rule as the max scores (|gpu - oracle| <= 1e-5 *
max(1, |oracle|)); selections may swap blocks whose oracle scores lie within
that band of the k-th selected score (2e-5 absolute near zero, where the
score tolerance is absolute)."""

import numpy as np
import pytest
import torch

import oracle
import parity
from synth import generate, host_view

pytestmark = pytest.mark.gpu

ABS_BAND = 2 * parity.SCORE_RTOL


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_score_amd as m
    m.load()
    return m


def _dec(B, lens, Hq=8, Hkv=2, Hidx=2, Di=128, topk=8, idx="bf16", q="bf16", kv="bf16"):
    return dict(kind="decode", B=B, seq_lens=list(lens), Hq=Hq, Hkv=Hkv, Hidx=Hidx, D=128,
                Di=Di, topk=topk, init=1, local=2, q=q, kv=kv, idx=idx)


def _pre(n_new, prefix, Hq=8, Hkv=2, Hidx=2, Di=128, topk=8):
    return dict(kind="prefill", B=len(n_new), n_new=list(n_new), prefix=list(prefix), Hq=Hq,
                Hkv=Hkv, Hidx=Hidx, D=128, Di=Di, topk=topk, init=1, local=2, q="bf16",
                kv="bf16", idx="bf16")


def _check(inp, g, spec, positions):
    f32 = spec.get("q", "bf16") == "f32"
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    parity.check_scores(parity.to_np(g["scores"]), ora_scores)
    gsel, gcnt = parity.to_np(g["sel"]), parity.to_np(g["cnt"])
    parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, positions, spec["init"],
                           spec["local"], abs_band=ABS_BAND)
    assert np.array_equal(parity.to_np(g["sel2"]), gsel)
    assert np.array_equal(parity.to_np(g["cnt2"]), gcnt)
    ora_out, ora_lse = oracle.attend(inp, gsel, gcnt)
    parity.check_output(parity.to_np(g["out"]), ora_out, f32)
    parity.check_lse(parity.to_np(g["lse"]), ora_lse, f32)


DECODE = {
    "ragged": _dec(5, [1, 127, 129, 1000, 9000]),
    "with_empty_di64": _dec(3, [0, 300, 5000], Hq=16, Hkv=4, Hidx=2, Di=64, topk=4),
    "idx_f32": _dec(3, [1500, 4000, 9000], idx="f32", q="f32", kv="f32"),
    "long_rows": _dec(2, [150001, 3000], Hq=8, Hkv=1, Hidx=1, topk=16),
}


@pytest.mark.parametrize("st", ["mean", "lse"])
@pytest.mark.parametrize("name", list(DECODE))
def test_decode_score_types(msa, name, st):
    spec = dict(DECODE[name], score_type=st)
    seed = 1400 + sorted(DECODE).index(name)
    print(f"[score_types_decode] {name} {st} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_decode(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, return_selection=True)
    scores = msa.block_score(cfg, case.idx_q, case.idx_k_pool, case.block_table, case.seq_lens)
    sel2, cnt2 = msa.select_blocks(cfg, scores, case.seq_lens)
    torch.cuda.synchronize()
    inp = host_view(case)
    assert inp["score_type"] == st
    _check(inp, dict(out=out, lse=lse, sel=sel, cnt=cnt, scores=scores, sel2=sel2, cnt2=cnt2),
           spec, oracle.query_positions(inp["seq_lens"], None))


@pytest.mark.parametrize("st", ["mean", "lse"])
def test_decode_score_types_with_index_value(msa, st):
    """The index scan fused with the index-value branch scores blocks the same
    way: the selection and output equal those of the branch switched off, and
    idx_out matches the oracle."""
    spec = dict(_dec(4, [1, 300, 5000, 20000], Hq=16, Hkv=2, Hidx=2), score_type=st,
                idx_value=True)
    print(f"[score_types_iv] {st}", flush=True)
    case = generate(spec, 1410, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    off = msa.MsaConfig.from_spec(dict(spec, idx_value=False))
    out, lse, sel, cnt, idx_out = msa.sparse_decode(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, return_selection=True, idx_v_pool=case.idx_v_pool)
    out0, lse0, sel0, cnt0 = msa.sparse_decode(
        off, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, return_selection=True)
    torch.cuda.synchronize()
    for a, b in ((out, out0), (lse, lse0), (sel, sel0), (cnt, cnt0)):
        assert torch.equal(a, b)
    inp = host_view(case)
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    parity.check_selection(parity.to_np(sel), parity.to_np(cnt), ora_scores, ora_sel, ora_cnt,
                           oracle.query_positions(inp["seq_lens"], None), spec["init"],
                           spec["local"], abs_band=ABS_BAND)
    ref, _ = oracle.index_value_attention(inp)
    parity.check_output(parity.to_np(idx_out).reshape(ref.shape), ref, False)


PREFILL = {
    # long chunks: the causal GEMM scoring (key-major attention)
    "key_major": _pre([300, 200], [1000, 0]),
    "ragged_empty": _pre([0, 257, 129], [500, 0, 3000], Hq=16, Hkv=2, Hidx=1),
    "di64": _pre([300, 129], [2000, 700], Hq=16, Hkv=1, Hidx=1, Di=64, topk=4),
    # short chunks: the multi-query page scan
    "short_chunks": _pre([4, 1, 3, 8], [30000, 999, 5000, 127], Hq=16, Hkv=2, Hidx=2),
}


@pytest.mark.parametrize("st", ["mean", "lse"])
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_score_types(msa, name, st):
    spec = dict(PREFILL[name], score_type=st)
    seed = 1420 + sorted(PREFILL).index(name)
    print(f"[score_types_prefill] {name} {st} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_prefill(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, case.cu_seqlens_q, return_selection=True)
    scores = msa.block_score(cfg, case.idx_q, case.idx_k_pool, case.block_table, case.seq_lens,
                             cu_seqlens_q=case.cu_seqlens_q)
    sel2, cnt2 = msa.select_blocks(cfg, scores, case.seq_lens, cu_seqlens_q=case.cu_seqlens_q)
    torch.cuda.synchronize()
    inp = host_view(case)
    _check(inp, dict(out=out, lse=lse, sel=sel, cnt=cnt, scores=scores, sel2=sel2, cnt2=cnt2),
           spec, oracle.query_positions(inp["seq_lens"], inp["cu_seqlens_q"]))
