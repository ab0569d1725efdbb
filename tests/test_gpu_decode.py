"""GPU parity of the decode path (score, select, split-K attend, combine)
against the fp64 oracle, through the C ABI."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import parity
from synth import WORKLOAD_SEEDS, generate, host_view, workload

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_score_amd as m
    m.load()
    return m


def _spec(B, lens, Hq=8, Hkv=2, Hidx=1, Di=128, topk=4, init=1, local=2, q="bf16",
          kv="bf16", idx="bf16", scale=None):
    s = dict(kind="decode", B=B, seq_lens=list(lens), Hq=Hq, Hkv=Hkv, Hidx=Hidx, D=128, Di=Di,
             topk=topk, init=init, local=local, q=q, kv=kv, idx=idx)
    if kv.startswith("fp8"):
        s.update(k_scale=1.0 / 16 if scale is None else scale[0],
                 v_scale=1.0 / 16 if scale is None else scale[1])
    return s


SMALL = {
    "cfg_b2_l2048": workload("decode_b2_l2048"),
    "ragged": _spec(5, [1, 127, 128, 129, 1000]),
    "with_empty": _spec(3, [0, 300, 5000], Hq=16, Hkv=4, Hidx=2),
    "dense_equiv": _spec(2, [2000, 4480], Hq=16, Hkv=2, Hidx=2, topk=32),
    "g16": _spec(2, [3000, 9000], Hq=16, Hkv=1, Hidx=1, topk=8),
    "g1": _spec(3, [700, 2100, 6000], Hq=2, Hkv=2, Hidx=2, topk=4),
    "g2_shared_idx": _spec(2, [5000, 9000], Hq=4, Hkv=2, Hidx=1, topk=8),
    "idx_f32_di64": _spec(3, [1500, 4000, 8000], Di=64, idx="f32", topk=8),
    "f32_path": _spec(3, [1500, 4000, 9000], Hq=8, Hkv=2, Hidx=2, q="f32", kv="f32", idx="f32",
                      topk=8),
    "fp8_small": _spec(3, [3000, 7000, 12345], Hq=16, Hkv=2, Hidx=2, kv="fp8", topk=8),
    "fp8_odd_scales": _spec(2, [4000, 6000], Hq=8, Hkv=1, Hidx=1, kv="fp8", topk=4,
                            scale=(0.37, 0.11)),
    "topk16_init0_local0": _spec(2, [9000, 20000], Hq=8, Hkv=1, Hidx=1, topk=16, init=0,
                                 local=0),
    "topk32_init3_local3": _spec(2, [20000, 30000], Hq=8, Hkv=2, Hidx=2, topk=32, init=3,
                                 local=3),
    # rows of more than 1024 blocks: the workgroup radix select (inside the
    # attention workgroups and in the standalone select kernel)
    "long_rows": _spec(2, [200000, 150001], Hq=8, Hkv=1, Hidx=1, topk=16),
}


def _run(msa, spec, seed, max_blocks=None, stream=None):
    case = generate(spec, seed, device="cuda", max_blocks=max_blocks)
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_decode(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, return_selection=True, stream=stream)
    scores = msa.block_score(cfg, case.idx_q, case.idx_k_pool, case.block_table, case.seq_lens,
                             stream=stream)
    sel2, cnt2 = msa.select_blocks(cfg, scores, case.seq_lens, stream=stream)
    out3, lse3 = msa.sparse_attend(cfg, case.q, case.k_pool, case.v_pool, case.block_table,
                                   case.seq_lens, sel, cnt, stream=stream)
    torch.cuda.synchronize()
    return case, cfg, dict(out=out, lse=lse, sel=sel, cnt=cnt, scores=scores, sel2=sel2,
                           cnt2=cnt2, out3=out3, lse3=lse3)


def _compare(inp, g, spec, rows=None):
    """Oracle on `inp`; rows restricts the check to some sequences (decode: token == seq)."""
    f32 = spec.get("q", "bf16") == "f32"
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    pos = oracle.query_positions(inp["seq_lens"], None)
    rows = list(range(len(pos))) if rows is None else rows
    gs = parity.to_np(g["scores"])
    parity.check_scores(gs[rows], ora_scores[rows])
    gsel, gcnt = parity.to_np(g["sel"]), parity.to_np(g["cnt"])
    nband = parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, pos,
                                   spec["init"], spec["local"], rows=rows)
    # the standalone select over the standalone scores agrees with the one the
    # attention workgroups run inside msa_sparse_decode
    assert np.array_equal(parity.to_np(g["sel2"])[rows], gsel[rows])
    assert np.array_equal(parity.to_np(g["cnt2"])[rows], gcnt[rows])
    # oracle attention over the GPU's own selection
    ora_out, ora_lse = oracle.attend(inp, gsel, gcnt)
    go = parity.to_np(g["out"])
    err = parity.check_output(go[rows], ora_out[rows], f32)
    parity.check_lse(parity.to_np(g["lse"])[rows], ora_lse[rows], f32)
    # step 3 alone, over that selection, reproduces msa_sparse_decode bit for bit
    assert torch.equal(g["out3"], g["out"])
    assert torch.equal(g["lse3"], g["lse"])
    return err, nband


@pytest.mark.parametrize("fmt", ["fp8", "fp8_e5m2"])
def test_fp8_dequant_all_codes(msa, fmt):
    """The loaders' conversion of all 256 codes (and a ragged count of 251)
    against the oracle's tables from the format definitions."""
    table = oracle.fp8_e4m3fn_table() if fmt == "fp8" else oracle.fp8_e5m2_table()
    for n in (256, 251):
        codes = torch.arange(n, dtype=torch.int32).to(torch.uint8).cuda()
        for scale in (1.0, 1.0 / 16, 0.37):
            got = msa.fp8_dequant(codes, scale, fmt=fmt).cpu().numpy().astype(np.float64)
            with np.errstate(invalid="ignore"):
                ref = table[:n] * np.float32(scale).astype(np.float64)
            ref = ref.astype(np.float32).astype(np.float64)   # the loader multiplies in fp32
            nan = np.isnan(ref)
            assert np.array_equal(np.isnan(got), nan)
            assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_small(msa, name):
    spec = SMALL[name]
    seed = 77 + sorted(SMALL).index(name)
    print(f"[decode_small] {name} seed={seed}", flush=True)
    case, cfg, g = _run(msa, spec, seed)
    err, nband = _compare(host_view(case), g, spec)
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


def test_decode_extra_table_columns(msa):
    """max_blocks larger than any sequence needs; unused entries are -1."""
    spec = _spec(3, [900, 5000, 2200], Hq=8, Hkv=2, Hidx=2, topk=4)
    case, cfg, g = _run(msa, spec, 5, max_blocks=97)
    _compare(host_view(case), g, spec)
    s = parity.to_np(g["scores"])
    assert s.shape[2] == 97 and np.isneginf(s[:, :, 40:]).all()


def test_decode_on_side_stream(msa):
    spec = SMALL["ragged"]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        case, cfg, g = _run(msa, spec, 9, stream=st)
    st.synchronize()
    _compare(host_view(case), g, spec)


def test_decode_deterministic(msa):
    spec = _spec(4, [30000, 12000, 64000, 5000], Hq=16, Hkv=2, Hidx=2, topk=16)
    case = generate(spec, 123, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    ws = msa.alloc_workspace(msa.decode_workspace_size(cfg, 4, case.max_blocks), "cuda")
    runs = []
    for _ in range(3):
        runs.append(msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                      case.idx_k_pool, case.block_table, case.seq_lens,
                                      workspace=ws, return_selection=True))
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def _golden_cases():
    with open(os.path.join(GOLDEN, "planted_selection.json")) as f:
        return json.load(f)["cases"]


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("case", [c for c in _golden_cases() if c["topk"] in (4, 8, 16, 32)],
                         ids=lambda c: c["name"])
def test_planted_selection_exact(msa, case):
    """Planted scores are exact in float32 as well: selection must match exactly.
    (Cases with a top-k outside the supported set pin only the oracle.)"""
    nb, tail, Di = case["nb"], case["tail"], 64
    L = (nb - 1) * 128 + tail
    P = nb + 3
    g = torch.Generator().manual_seed(nb)
    perm = torch.randperm(P, generator=g)
    bt = perm[:nb].to(torch.int32)[None, :]
    ik = torch.randn((P, 1, 128, Di), generator=g)
    ik[:, :, :, 0] = -1000.0
    scores = [(-0.0 if s == "-0" else float(s)) for s in case["scores"]]
    for j in range(nb):
        valid = 128 if j < nb - 1 else tail
        ik[bt[0, j], 0, (37 * j + 11) % valid, 0] = scores[j]
    if "decoy" in case and tail < 128:
        ik[bt[0, nb - 1], 0, tail:, 0] = case["decoy"]
    iq = torch.zeros((1, 1, Di))
    iq[0, 0, 0] = 1.0
    cfg = msa.MsaConfig(num_q_heads=1, num_kv_heads=1, num_idx_heads=1, idx_dim=Di,
                        topk=case["topk"], init_blocks=case["init"],
                        local_blocks=case["local"])
    sl = torch.tensor([L], dtype=torch.int32).cuda()
    s = msa.block_score(cfg, iq.to(torch.bfloat16).cuda(), ik.to(torch.bfloat16).cuda(),
                        bt.cuda(), sl)
    sel, cnt = msa.select_blocks(cfg, s, sl)
    torch.cuda.synchronize()
    got = s.cpu()[0, 0, :nb].tolist()
    assert got == scores
    assert sel.cpu()[0, 0, : int(cnt.cpu()[0, 0])].tolist() == case["expected"]


@pytest.mark.parametrize("width", [0, 300, 1100], ids=["mb_nb", "mb300", "mb1100"])
@pytest.mark.parametrize("case", [c for c in _golden_cases() if c["topk"] in (4, 8, 16, 32)],
                         ids=lambda c: c["name"])
def test_planted_selection_in_decode(msa, case, width):
    """The same planted rows through msa_sparse_decode, whose attention
    workgroups select in-kernel: with the table as wide as the row, 300 wide
    (a row fetched 16 slots per lane, selected as 4) and 1100 wide (past the
    one-wave rows, the row fetched after the length).  Unused table columns
    hold -1."""
    nb, tail, Di = case["nb"], case["tail"], 64
    L = (nb - 1) * 128 + tail
    MB = max(width, nb)
    P = nb + 3
    g = torch.Generator().manual_seed(nb)
    perm = torch.randperm(P, generator=g)
    bt = torch.full((1, MB), -1, dtype=torch.int32)
    bt[0, :nb] = perm[:nb].to(torch.int32)
    ik = torch.randn((P, 1, 128, Di), generator=g)
    ik[:, :, :, 0] = -1000.0
    scores = [(-0.0 if s == "-0" else float(s)) for s in case["scores"]]
    for j in range(nb):
        valid = 128 if j < nb - 1 else tail
        ik[bt[0, j], 0, (37 * j + 11) % valid, 0] = scores[j]
    if "decoy" in case and tail < 128:
        ik[bt[0, nb - 1], 0, tail:, 0] = case["decoy"]
    iq = torch.zeros((1, 1, Di))
    iq[0, 0, 0] = 1.0
    kp = torch.randn((P, 1, 128, 128), generator=g).to(torch.bfloat16).cuda()
    vp = torch.randn((P, 1, 128, 128), generator=g).to(torch.bfloat16).cuda()
    q = torch.randn((1, 1, 128), generator=g).to(torch.bfloat16).cuda()
    cfg = msa.MsaConfig(num_q_heads=1, num_kv_heads=1, num_idx_heads=1, idx_dim=Di,
                        topk=case["topk"], init_blocks=case["init"],
                        local_blocks=case["local"])
    sl = torch.tensor([L], dtype=torch.int32).cuda()
    _, _, sel, cnt = msa.sparse_decode(cfg, q, iq.to(torch.bfloat16).cuda(), kp, vp,
                                       ik.to(torch.bfloat16).cuda(), bt.cuda(), sl,
                                       return_selection=True)
    torch.cuda.synchronize()
    n = int(cnt.cpu()[0, 0])
    assert sel.cpu()[0, 0, :n].tolist() == case["expected"]
    assert (sel.cpu()[0, 0, n:] == -1).all()


@pytest.mark.parametrize("nb,topk,width,seed", [(257, 4, 257, 0), (300, 16, 305, 1),
                                                (600, 32, 600, 2), (1024, 32, 1024, 3)])
def test_long_row_ties(msa, nb, topk, width, seed):
    """Rows of 257 to 1024 blocks (one wave, 16 slots per lane) whose scores
    come from eight values, so that many blocks tie at the cutoff and -0 meets
    +0: the selection made inside msa_sparse_decode's attention workgroups
    and the one of msa_select_blocks must both be the oracle's (score desc,
    lower block first on ties, forced init and local blocks added).  Table
    columns past the row hold -1."""
    print(f"[long_row_ties] nb={nb} topk={topk} width={width} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    vals = np.array([-3.0, -2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0])
    scores = vals[rng.integers(0, len(vals), nb)]
    tail = 1 + int(rng.integers(0, 128))
    L = (nb - 1) * 128 + tail
    P, Di, init, local = nb + 3, 64, 1, 2
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(P, generator=g)
    bt = torch.full((1, width), -1, dtype=torch.int32)
    bt[0, :nb] = perm[:nb].to(torch.int32)
    ik = torch.zeros((P, 1, 128, Di))
    ik[:, :, :, 0] = -1000.0
    for j in range(nb):
        valid = 128 if j < nb - 1 else tail
        ik[bt[0, j], 0, (37 * j + 11) % valid, 0] = float(scores[j])
    iq = torch.zeros((1, 1, Di))
    iq[0, 0, 0] = 1.0
    kp = torch.randn((P, 1, 128, 128), generator=g).to(torch.bfloat16).cuda()
    vp = torch.randn((P, 1, 128, 128), generator=g).to(torch.bfloat16).cuda()
    q = torch.randn((1, 1, 128), generator=g).to(torch.bfloat16).cuda()
    cfg = msa.MsaConfig(num_q_heads=1, num_kv_heads=1, num_idx_heads=1, idx_dim=Di, topk=topk,
                        init_blocks=init, local_blocks=local)
    sl = torch.tensor([L], dtype=torch.int32).cuda()
    ikd, iqd, btd = ik.to(torch.bfloat16).cuda(), iq.to(torch.bfloat16).cuda(), bt.cuda()
    expected = oracle.select_for_query(scores, nb, topk, init, local)
    _, _, sel, cnt = msa.sparse_decode(cfg, q, iqd, kp, vp, ikd, btd, sl, return_selection=True)
    s = msa.block_score(cfg, iqd, ikd, btd, sl)
    sel2, cnt2 = msa.select_blocks(cfg, s, sl)
    torch.cuda.synchronize()
    assert [float(x) for x in s.cpu()[0, 0, :nb]] == [float(x) for x in scores]
    for name, sl_, cn in (("decode", sel, cnt), ("select_blocks", sel2, cnt2)):
        n = int(cn.cpu()[0, 0])
        assert sl_.cpu()[0, 0, :n].tolist() == expected, name
        assert (sl_.cpu()[0, 0, n:] == -1).all(), name


# ----------------------------------------------------------- full sizes

FULL = ["decode_b32_l32k", "decode_b64_lvar", "decode_fp8_b32_l64k"]


def _sub_input(case, rows):
    """Host copy of sequences ``rows`` only (their pages, queries, tables and
    lengths), so the oracle scores nothing else."""
    bt = case.block_table.cpu().numpy()
    pages = np.unique(bt[rows].reshape(-1))
    inp = host_view(case, pages=pages[pages >= 0])
    for key in ("q", "idx_q", "block_table", "seq_lens"):
        inp[key] = inp[key][rows]
    return inp


@pytest.mark.parametrize("name", FULL)
def test_decode_full_size(msa, name):
    """The full workload in the launch configuration the benchmark times; the
    oracle checks every sequence (all heads and blocks), eight at a time."""
    spec = workload(name)
    seed = WORKLOAD_SEEDS[name]
    print(f"[decode_full] {name} seed={seed}", flush=True)
    case, cfg, g = _run(msa, spec, seed)
    B = case.B
    worst = [0.0, 0.0]
    nband = 0
    for r0 in range(0, B, 8):
        rows = list(range(r0, min(B, r0 + 8)))
        sub = {k: (v[rows] if k in ("out", "lse", "sel", "cnt", "scores", "sel2", "cnt2",
                                    "out3", "lse3") else v) for k, v in g.items()}
        err, nb_ = _compare(_sub_input(case, rows), sub, spec)
        worst = [max(worst[0], err[0]), max(worst[1], err[1])]
        nband += nb_
    print(f"  all {B} sequences: max {worst[0]:.3g} worst mean {worst[1]:.3g} "
          f"band-rows {nband}", flush=True)
    cnt = parity.to_np(g["cnt"])
    kmax = spec["topk"] + spec["init"] + spec["local"]
    nb = (case.seq_lens.cpu().numpy() + 127) // 128
    assert (cnt == np.minimum(nb, kmax)[:, None]).all()


def test_decode_repeats_match_composition(msa):
    """Split partials pass between workgroups through atomic tickets, and every
    split workgroup re-runs its row's selection; repeated calls must agree bit
    for bit with each other and with the composition block_score ->
    select_blocks -> sparse_attend."""
    spec = _spec(8, [131072, 70000, 4096, 33000, 100000, 129, 65536, 9000], Hq=16, Hkv=2,
                 Hidx=2, topk=32, init=1, local=2)
    case = generate(spec, 321, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    ws = msa.alloc_workspace(msa.decode_workspace_size(cfg, case.B, case.max_blocks), "cuda")
    scores = msa.block_score(cfg, case.idx_q, case.idx_k_pool, case.block_table, case.seq_lens)
    sel_u, cnt_u = msa.select_blocks(cfg, scores, case.seq_lens)
    out_u, lse_u = msa.sparse_attend(cfg, case.q, case.k_pool, case.v_pool, case.block_table,
                                     case.seq_lens, sel_u, cnt_u, workspace=ws)
    out_u, lse_u = out_u.clone(), lse_u.clone()
    for i in range(40):
        out, lse, sel, cnt = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool,
                                               case.v_pool, case.idx_k_pool, case.block_table,
                                               case.seq_lens, workspace=ws,
                                               return_selection=True)
        assert torch.equal(sel, sel_u) and torch.equal(cnt, cnt_u), f"call {i}: selection"
        assert torch.equal(out, out_u) and torch.equal(lse, lse_u), f"call {i}: output"


def test_decode_maximum_sizes(msa):
    """The largest supported shapes: a sequence of 8192 blocks (1M tokens, the
    max_blocks limit) beside a short one, and the largest selection (topk 32
    with 64 init and 64 local blocks, 160 slots), so a row is cut into more
    splits than the one-round-trip combine takes."""
    spec = _spec(2, [8192 * 128, 5000], Hq=8, Hkv=1, Hidx=1, Di=64, topk=32, init=64, local=64)
    print("[decode_max] seed=31", flush=True)
    case, cfg, g = _run(msa, spec, 31)
    assert case.max_blocks == 8192
    err, nband = _compare(host_view(case), g, spec)
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


E5M2 = {
    "e5m2_small": _spec(3, [3000, 7000, 12345], Hq=16, Hkv=2, Hidx=2, kv="fp8_e5m2", topk=8),
    "e5m2_odd_scales_long": _spec(2, [40000, 150000], Hq=8, Hkv=1, Hidx=1, kv="fp8_e5m2",
                                  topk=16, scale=(0.37, 0.11)),
}


@pytest.mark.parametrize("name", list(E5M2))
def test_decode_e5m2(msa, name):
    """fp8-e5m2 K/V pools (the sglang page's other fp8 cache format), dequantised
    on load; the second case has a row of more than 1024 blocks."""
    spec = E5M2[name]
    seed = 700 + sorted(E5M2).index(name)
    print(f"[decode_e5m2] {name} seed={seed}", flush=True)
    case, cfg, g = _run(msa, spec, seed)
    err, nband = _compare(host_view(case), g, spec)
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


BUDGET = {
    "budget_g8": dict(_spec(3, [5000, 30000, 700], Hq=16, Hkv=2, Hidx=2, topk=16),
                      forced_in_budget=True),
    # |F| = 6 > topk = 4: the selection is the forced blocks alone; the long row
    # takes the workgroup radix select
    "budget_forced_exceed": dict(_spec(2, [9000, 140000], Hq=8, Hkv=1, Hidx=1, topk=4, init=3,
                                       local=3), forced_in_budget=True),
}


@pytest.mark.parametrize("name", list(BUDGET))
def test_decode_forced_in_budget(msa, name):
    """The other reading of the budget: forced blocks count inside topk."""
    spec = BUDGET[name]
    seed = 720 + sorted(BUDGET).index(name)
    print(f"[decode_budget] {name} seed={seed}", flush=True)
    case, cfg, g = _run(msa, spec, seed)
    assert cfg.forced_in_budget
    err, nband = _compare(host_view(case), g, spec)
    lens = case.seq_lens.cpu().numpy()
    nb = (lens + 127) // 128
    F = np.array([len(oracle.forced_blocks(int(n), spec["init"], spec["local"])) for n in nb])
    want = np.minimum(nb, np.maximum(spec["topk"], F))
    assert (parity.to_np(g["cnt"]) == want[:, None]).all()
    print(f"  max {err[0]:.3g} mean {err[1]:.3g} band-rows {nband}", flush=True)


def test_sparse_equals_dense_over_compacted_table(msa):
    """The library's sparse decode against its own decode over a page table
    compacted to the selected blocks, where every block is selected (the
    sglang page's dense-sparse form): the same attention, summed in another
    order, so within the parity bounds of each other and of the oracle."""
    spec = _spec(4, [33000, 5000, 129, 20000], Hq=16, Hkv=2, Hidx=1, topk=16)
    print("[compacted] seed=731", flush=True)
    case, cfg, g = _run(msa, spec, 731)
    _compare(host_view(case), g, spec)
    sel, cnt = parity.to_np(g["sel"]), parity.to_np(g["cnt"])
    lens = case.seq_lens.cpu().numpy()
    bt = case.block_table.cpu().numpy()
    K = sel.shape[2]
    bt_c = np.full((case.B, K), -1, dtype=np.int32)
    lens_c = np.zeros(case.B, dtype=np.int32)
    for b in range(case.B):
        c = int(cnt[b, 0])
        bt_c[b, :c] = bt[b, sel[b, 0, :c]]
        nb = (int(lens[b]) + 127) // 128
        assert sel[b, 0, c - 1] == nb - 1
        lens_c[b] = 128 * (c - 1) + (int(lens[b]) - 128 * (nb - 1))
    dense_cfg = msa.MsaConfig.from_spec(dict(spec, topk=32))  # every compacted block is kept
    out_c = msa.sparse_decode(dense_cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                              case.idx_k_pool, torch.from_numpy(bt_c).cuda(),
                              torch.from_numpy(lens_c).cuda())
    torch.cuda.synchronize()
    d = (out_c.float() - g["out"].float()).abs()
    assert d.max().item() <= parity.BF16_MAX and d.mean().item() <= parity.BF16_MEAN


def test_decode_all_sequences_empty(msa):
    """Every sequence of the batch has length 0: zeros, lse -inf, empty selections."""
    spec = _spec(3, [0, 0, 0], Hq=16, Hkv=2, Hidx=2, topk=8)
    print("[decode_empty] seed=741", flush=True)
    case = generate(spec, 741, device="cuda", max_blocks=4)
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                           case.idx_k_pool, case.block_table, case.seq_lens,
                                           return_selection=True)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
    assert (cnt == 0).all() and (sel == -1).all()
