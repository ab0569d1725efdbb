"""GPU parity of chunked prefill (causal index scoring on the matrix cores,
per-token selection, attention over each token's selection) against the fp64
oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import parity
from synth import WORKLOAD_SEEDS, generate, host_view, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_score_amd as m
    m.load()
    return m


def _spec(n_new, prefix, Hq=8, Hkv=2, Hidx=2, Di=128, topk=4, init=1, local=2, q="bf16",
          kv="bf16"):
    s = dict(kind="prefill", B=len(n_new), n_new=list(n_new), prefix=list(prefix), Hq=Hq,
             Hkv=Hkv, Hidx=Hidx, D=128, Di=Di, topk=topk, init=init, local=local, q=q, kv=kv,
             idx="bf16")
    if kv.startswith("fp8"):
        s.update(k_scale=1.0 / 16, v_scale=1.0 / 16)
    return s


SMALL = {
    "two_seqs": _spec([100, 300], [50, 1000]),
    "from_scratch_ragged": _spec([257, 1, 700], [0, 0, 130], Hq=4, Hkv=1, Hidx=1, topk=8),
    "empty_chunk": _spec([0, 200, 300], [500, 0, 3000], Hq=16, Hkv=2, Hidx=1, topk=8),
    "di64_g16": _spec([300, 129], [2000, 700], Hq=16, Hkv=1, Hidx=1, Di=64, topk=4, init=2,
                      local=1),
    "fp8": _spec([260, 100], [4000, 1500], Hq=16, Hkv=2, Hidx=2, kv="fp8", topk=8),
    "f32_qkv": _spec([150, 200], [1000, 2500], Hq=8, Hkv=2, Hidx=2, q="f32", kv="f32", topk=8),
    "topk32_long": _spec([512], [8000], Hq=16, Hkv=2, Hidx=2, topk=32, init=1, local=2),
    # one q head per kv head: 256-token tiles, lists longer than a tile
    "g1_long_lists": _spec([700, 300], [300, 0], Hq=2, Hkv=2, Hidx=1, topk=4, init=1,
                           local=2),
    "g2": _spec([400], [1200], Hq=4, Hkv=2, Hidx=2, topk=8),
    # a prefix of more than 1024 blocks: the workgroup radix select per token
    "long_prefix": _spec([40], [160000], Hq=8, Hkv=1, Hidx=1, topk=8),
}


def _run(msa, case, spec):
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_prefill(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, case.cu_seqlens_q, return_selection=True)
    scores = msa.block_score(cfg, case.idx_q, case.idx_k_pool, case.block_table, case.seq_lens,
                             cu_seqlens_q=case.cu_seqlens_q)
    sel2, cnt2 = msa.select_blocks(cfg, scores, case.seq_lens, cu_seqlens_q=case.cu_seqlens_q)
    torch.cuda.synchronize()
    return dict(out=out, lse=lse, sel=sel, cnt=cnt, scores=scores, sel2=sel2, cnt2=cnt2)


def _compare(inp, g, spec, rows):
    f32 = spec.get("q", "bf16") == "f32"
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    pos = oracle.query_positions(inp["seq_lens"], inp.get("cu_seqlens_q"), inp.get("positions"))
    gs = parity.to_np(g["scores"])[rows]
    parity.check_scores(gs, ora_scores)
    gsel, gcnt = parity.to_np(g["sel"])[rows], parity.to_np(g["cnt"])[rows]
    nband = parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, pos,
                                   spec["init"], spec["local"])
    assert np.array_equal(parity.to_np(g["sel2"])[rows], gsel)
    assert np.array_equal(parity.to_np(g["cnt2"])[rows], gcnt)
    ora_out, ora_lse = oracle.attend(inp, gsel, gcnt)
    err = parity.check_output(parity.to_np(g["out"])[rows], ora_out, f32)
    parity.check_lse(parity.to_np(g["lse"])[rows], ora_lse, f32)
    return err, nband


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_small(msa, name):
    spec = SMALL[name]
    seed = 500 + sorted(SMALL).index(name)
    print(f"[prefill_small] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    g = _run(msa, case, spec)
    rows = np.arange(case.T)
    err, nband = _compare(host_view(case), g, spec, rows)
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


# The forced blocks (init and local) of long chunks run query-major over
# groups of consecutive tokens, one merged partial per token in its first
# forced slot: no init blocks (that slot is the first local one), no local
# blocks, every visible block forced, none forced, and groups that straddle a
# block boundary (prefixes off the 128 grid).
FORCED_SPLIT = {
    "init0_local2": _spec([300, 200], [1000, 77], Hq=8, Hkv=2, Hidx=2, topk=4, init=0, local=2),
    "init2_local0": _spec([300], [2000], Hq=8, Hkv=1, Hidx=1, topk=4, init=2, local=0),
    "all_forced": _spec([300, 50], [0, 100], Hq=8, Hkv=2, Hidx=1, topk=4, init=3, local=3),
    "none_forced": _spec([200], [1500], Hq=8, Hkv=2, Hidx=2, topk=8, init=0, local=0),
    "init3_local4_g16": _spec([400, 33], [5000, 1234], Hq=16, Hkv=1, Hidx=1, topk=8, init=3,
                              local=4),
}


@pytest.mark.parametrize("name", list(FORCED_SPLIT))
def test_prefill_forced_split(msa, name):
    spec = FORCED_SPLIT[name]
    seed = 2100 + sorted(FORCED_SPLIT).index(name)
    print(f"[prefill_forced_split] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


# Multi-token decode (speculative verification): a few new tokens per
# sequence over long contexts, causal among themselves, each with its own
# selection -- the prefill call with short chunks.
VERIFY = {
    "q4_long": _spec([4] * 6, [30000, 999, 5000, 12000, 127, 70000], Hq=16, Hkv=2, Hidx=2,
                     topk=16),
    "ragged_q": _spec([1, 2, 3, 5, 8], [20000, 4000, 300, 9000, 130], Hq=8, Hkv=2, Hidx=1,
                      topk=8),
    "fp8_q3": _spec([3, 3, 3], [40000, 7000, 16000], Hq=16, Hkv=2, Hidx=2, kv="fp8", topk=32),
    # two query groups per scan pass, an empty chunk, a row of more than 1024 blocks
    "groups_empty_long": _spec([7, 0, 9, 1], [3000, 500, 140000, 20], Hq=16, Hkv=1, Hidx=1,
                               Di=64, topk=8),
}


@pytest.mark.parametrize("name", list(VERIFY))
def test_multi_token_decode(msa, name):
    spec = VERIFY[name]
    seed = 900 + sorted(VERIFY).index(name)
    print(f"[verify] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


# Batches of more than a wave's worth of sequences: the per-token selection
# finds a token's sequence by a search over the offsets instead of one ballot
# (64 sequences is the last batch on the ballot path).  Lengths and new-token
# counts cycle through patterns that include empty sequences and chunks.
MANY_SEQS = {
    "short_70": _spec([i % 4 for i in range(70)], [(i * 997) % 3000 for i in range(70)],
                      Hq=8, Hkv=1, Hidx=1, topk=4),
    "short_64": _spec([1 + i % 3 for i in range(64)], [(i * 331) % 2000 for i in range(64)],
                      Hq=8, Hkv=1, Hidx=1, topk=4),
    "key_major_66": _spec([20 + i % 7 for i in range(66)], [(i * 53) % 700 for i in range(66)],
                          Hq=8, Hkv=2, Hidx=2, topk=4),
}


@pytest.mark.parametrize("name", list(MANY_SEQS))
def test_many_sequences(msa, name):
    spec = MANY_SEQS[name]
    seed = 960 + list(MANY_SEQS).index(name)
    print(f"[many_seqs] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  T={case.T} max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


def test_single_token_chunks_match_decode(msa):
    """A prefill of one new token per sequence is a decode step: the same
    selection, bit for bit, and outputs that agree within the parity bounds
    (the two paths split the keys differently)."""
    spec = _spec([1] * 5, [33000, 4095, 128, 9000, 1], Hq=16, Hkv=2, Hidx=2, topk=16)
    print("[verify_vs_decode] seed=950", flush=True)
    case = generate(spec, 950, device="cuda")
    g = _run(msa, case, spec)
    cfg = msa.MsaConfig.from_spec(spec)
    out_d, lse_d, sel_d, cnt_d = msa.sparse_decode(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, return_selection=True)
    torch.cuda.synchronize()
    assert torch.equal(sel_d, g["sel"]) and torch.equal(cnt_d, g["cnt"])
    d = (out_d.float() - g["out"].float()).abs()
    assert d.max().item() <= parity.BF16_MAX and d.mean().item() <= parity.BF16_MEAN
    err, _ = _compare(host_view(case), dict(g, out=out_d, lse=lse_d), spec, np.arange(case.T))
    print(f"  decode vs oracle: max {err[0]:.3g} mean {err[1]:.3g}", flush=True)


def test_prefill_full_size(msa):
    """The full chunked-prefill workload (4 x 4096 new tokens over 16384) in
    the launch configuration the benchmark times: the oracle checks the scores
    and the selection of every token, and the output of every fourth token of
    each sequence plus every token at a block boundary (the first and last of
    each 128-token block)."""
    name = "prefill_4x4096_p16k"
    spec = workload(name)
    case = generate(spec, WORKLOAD_SEEDS[name], device="cuda")
    print(f"[prefill_full] {name}", flush=True)
    g = _run(msa, case, spec)
    inp = host_view(case)
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    pos = oracle.query_positions(inp["seq_lens"], inp["cu_seqlens_q"])
    parity.check_scores(parity.to_np(g["scores"]), ora_scores)
    gsel, gcnt = parity.to_np(g["sel"]), parity.to_np(g["cnt"])
    nband = parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, pos,
                                   spec["init"], spec["local"])
    assert np.array_equal(parity.to_np(g["sel2"]), gsel)
    assert np.array_equal(parity.to_np(g["cnt2"]), gcnt)
    print(f"  scores and selection of all {case.T} tokens; band-rows {nband}", flush=True)
    rows = np.array([t for t, (b, p) in enumerate(pos)
                     if t % 4 == 0 or p % 128 in (0, 127)])
    sub = dict(inp)
    sub["q"] = inp["q"][rows]
    sub["positions"] = [pos[t] for t in rows]
    ora_out, ora_lse = oracle.attend(sub, gsel[rows], gcnt[rows])
    err = parity.check_output(parity.to_np(g["out"])[rows], ora_out, False)
    parity.check_lse(parity.to_np(g["lse"])[rows], ora_lse, False)
    print(f"  outputs of {len(rows)} tokens: max {err[0]:.3g} mean {err[1]:.3g}", flush=True)
    assert (gcnt == spec["topk"] + spec["init"] + spec["local"]).all()
    assert torch.isfinite(g["out"].float()).all()


def test_prefill_maximum_sizes(msa):
    """A prefix that fills the table (8192 blocks, the max_blocks limit) with
    the largest selection (160 slots: topk 32, 64 init, 64 local)."""
    spec = _spec([24, 100], [8192 * 128 - 24, 3000], Hq=8, Hkv=1, Hidx=1, Di=64, topk=32,
                 init=64, local=64)
    print("[prefill_max] seed=41", flush=True)
    case = generate(spec, 41, device="cuda")
    assert case.max_blocks == 8192
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


E5M2 = {
    "key_major": _spec([260, 100], [4000, 1500], Hq=16, Hkv=2, Hidx=2, kv="fp8_e5m2", topk=8),
    "short_chunks": _spec([3, 4, 1], [40000, 7000, 16000], Hq=16, Hkv=2, Hidx=2,
                          kv="fp8_e5m2", topk=32),
}


@pytest.mark.parametrize("name", list(E5M2))
def test_prefill_e5m2(msa, name):
    spec = E5M2[name]
    seed = 960 + sorted(E5M2).index(name)
    print(f"[prefill_e5m2] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


BUDGET = {
    "key_major": dict(_spec([300, 200], [5000, 2000], topk=8, init=2, local=2),
                      forced_in_budget=True),
    "short_forced_exceed": dict(_spec([4, 4, 2], [20000, 3000, 140000], Hq=8, Hkv=1, Hidx=1,
                                      topk=4, init=3, local=3), forced_in_budget=True),
}


@pytest.mark.parametrize("name", list(BUDGET))
def test_prefill_forced_in_budget(msa, name):
    spec = BUDGET[name]
    seed = 980 + sorted(BUDGET).index(name)
    print(f"[prefill_budget] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


def test_short_chunks_with_empty_sequences(msa):
    """Short chunks where some sequences have no tokens at all (length 0, no new
    tokens) and some chunks are empty."""
    spec = _spec([2, 0, 3, 0], [5000, 0, 300, 0], Hq=8, Hkv=2, Hidx=2, topk=8)
    print("[short_empty] seed=990", flush=True)
    case = generate(spec, 990, device="cuda")
    g = _run(msa, case, spec)
    err, nband = _compare(host_view(case), g, spec, np.arange(case.T))
    print(f"  max {err[0]:.3g} mean {err[1]:.3g}", flush=True)
