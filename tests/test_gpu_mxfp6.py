"""GPU parity of MX-fp6 K/V pools (OCP E2M3 codes with an E8M0 scale per 32
elements, widened on load by the gfx950 32-code scaled conversion) against
the fp64 oracle, through the C ABI: the loaders' conversion of every code,
decode, long and short prefill chunks, the full-size decode workload and the
append's quantise-on-store, byte for byte."""

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


def test_mxfp6_conversion_all_codes(msa):
    """Every code in every position of a group under several scale codes (and
    the NaN scale) against the oracle's tables; the loaders' bf16 products,
    times a float32 scale."""
    sc = np.array([127, 126, 130, 100, 160, 10, 240, 255, 127, 128, 120, 135, 90, 200, 127, 127],
                  dtype=np.uint8)
    n = 32 * len(sc)
    codes = (np.arange(n) * 5 + np.arange(n) // 64) % 64        # each code in many slots
    buf = torch.from_numpy(np.concatenate([oracle.fp6_pack(codes), sc])).cuda()
    tab, e8 = oracle.fp6_e2m3_table(), oracle.e8m0_table()
    for scale in (1.0, 0.37):
        got = msa.fp8_dequant(buf, scale, fmt="mxfp6").cpu().numpy().astype(np.float64)
        with np.errstate(invalid="ignore"):
            ref = (tab[codes] * np.repeat(e8[sc], 32)).astype(np.float32)
            ref = (ref * np.float32(scale)).astype(np.float64)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])


def _dec(B, lens, Hq=16, Hkv=2, Hidx=2, topk=8, ks=1.0, vs=1.0):
    return dict(kind="decode", B=B, seq_lens=list(lens), Hq=Hq, Hkv=Hkv, Hidx=Hidx, D=128,
                Di=128, topk=topk, init=1, local=2, q="bf16", kv="mxfp6", idx="bf16",
                k_scale=ks, v_scale=vs)


DECODE = {
    "ragged": _dec(5, [1, 127, 129, 1000, 9000]),
    "g8_long": _dec(2, [40000, 150001], Hq=8, Hkv=1, Hidx=1, topk=16),
    "g2_scales": _dec(3, [3000, 7000, 12345], Hq=4, Hkv=2, Hidx=1, topk=4, ks=0.5, vs=2.0),
}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_mxfp6(msa, name):
    spec = DECODE[name]
    seed = 1700 + sorted(DECODE).index(name)
    print(f"[mxfp6_decode] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                           case.idx_k_pool, case.block_table, case.seq_lens,
                                           return_selection=True)
    torch.cuda.synchronize()
    inp = host_view(case)
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    gsel, gcnt = parity.to_np(sel), parity.to_np(cnt)
    pos = oracle.query_positions(inp["seq_lens"], None)
    parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, pos, 1, 2)
    ora_out, ora_lse = oracle.attend(inp, gsel, gcnt)
    parity.check_output(parity.to_np(out), ora_out, False)
    parity.check_lse(parity.to_np(lse), ora_lse, False)


PREFILL = {
    "key_major": dict(kind="prefill", B=2, n_new=[300, 200], prefix=[1000, 0], Hq=16, Hkv=2,
                      Hidx=2, D=128, Di=128, topk=8, init=1, local=2, q="bf16", kv="mxfp6",
                      idx="bf16"),
    "short_chunks": dict(kind="prefill", B=3, n_new=[4, 1, 3], prefix=[30000, 999, 5000],
                         Hq=16, Hkv=2, Hidx=2, D=128, Di=128, topk=16, init=1, local=2,
                         q="bf16", kv="mxfp6", idx="bf16", k_scale=0.25, v_scale=4.0),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_mxfp6(msa, name):
    spec = PREFILL[name]
    seed = 1800 + sorted(PREFILL).index(name)
    print(f"[mxfp6_prefill] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    out, lse, sel, cnt = msa.sparse_prefill(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                            case.idx_k_pool, case.block_table, case.seq_lens,
                                            case.cu_seqlens_q, return_selection=True)
    torch.cuda.synchronize()
    inp = host_view(case)
    ora_scores = oracle.block_scores(inp)
    ora_sel, ora_cnt = oracle.select(inp, ora_scores)
    gsel, gcnt = parity.to_np(sel), parity.to_np(cnt)
    pos = oracle.query_positions(inp["seq_lens"], inp["cu_seqlens_q"])
    parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, pos, 1, 2)
    ora_out, ora_lse = oracle.attend(inp, gsel, gcnt)
    parity.check_output(parity.to_np(out), ora_out, False)
    parity.check_lse(parity.to_np(lse), ora_lse, False)


def test_decode_mxfp6_full_size(msa):
    """The 32 x 65536 decode workload with MX-fp6 pools: every sequence's
    selection and output against the oracle, eight sequences at a time."""
    name = "decode_mxfp6_b32_l64k"
    spec = workload(name)
    case = generate(spec, WORKLOAD_SEEDS[name], device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    print(f"[mxfp6_full] {name}", flush=True)
    out, lse, sel, cnt = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                           case.idx_k_pool, case.block_table, case.seq_lens,
                                           return_selection=True)
    torch.cuda.synchronize()
    bt = case.block_table.cpu().numpy()
    for r0 in range(0, case.B, 8):
        rows = list(range(r0, r0 + 8))
        pages = np.unique(bt[rows].reshape(-1))
        inp = host_view(case, pages=pages[pages >= 0])
        for key in ("q", "idx_q", "block_table", "seq_lens"):
            inp[key] = inp[key][rows]
        ora_scores = oracle.block_scores(inp)
        ora_sel, ora_cnt = oracle.select(inp, ora_scores)
        gsel, gcnt = parity.to_np(sel)[rows], parity.to_np(cnt)[rows]
        pos = oracle.query_positions(inp["seq_lens"], None)
        parity.check_selection(gsel, gcnt, ora_scores, ora_sel, ora_cnt, pos, 1, 2)
        ora_out, _ = oracle.attend(inp, gsel, gcnt)
        parity.check_output(parity.to_np(out)[rows], ora_out, False)


def test_append_mxfp6_bytes(msa):
    """Quantise-on-store into MX-fp6 pools: every byte of the pools equals the
    oracle's append (codes, scale codes, untouched slots), including a group
    of zeros, a group with a NaN, values needing the clamp at 7.5 and a group
    of exact midpoints between neighbouring codes (ties to the even code)."""
    spec = dict(kind="decode", B=2, seq_lens=[300, 500], Hq=8, Hkv=2, Hidx=2, D=128, Di=128,
                topk=4, init=1, local=2, q="bf16", kv="mxfp6", idx="bf16", k_scale=0.5,
                v_scale=2.0)
    case = generate(spec, 1900, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    T = 41
    g = torch.Generator(device="cpu").manual_seed(8)
    k_new = (torch.randn((T, 2, 128), generator=g) * 3).to(torch.bfloat16)
    v_new = torch.randn((T, 2, 128), generator=g).to(torch.bfloat16)
    k_new[0, 0, :32] = 0.0
    k_new[1, 1, 40] = float("nan")
    k_new[2, 0, 64:96] = torch.tensor([7.0, -7.9] + [0.001] * 30)
    # y = x / 0.5 lands on the E2M3 midpoints (scale 2^0: max |y| = 7.5)
    tab = oracle.fp6_e2m3_table()
    mids = [(tab[i] + tab[i + 1]) / 2 for i in range(31)] + [7.5]
    k_new[3, 1, 32:64] = torch.tensor(mids, dtype=torch.float64) * 0.5
    v_new[4, 0, 0:32] = -torch.tensor(mids, dtype=torch.float64) * 2.0
    ik_new = torch.randn((T, 2, 128), generator=g).to(torch.bfloat16)
    slots = torch.randperm(case.num_pages * 128, generator=g)[:T].to(torch.int64)
    slots[5] = -1
    before = host_view(case)
    msa.append_kv(cfg, k_new.cuda(), v_new.cuda(), ik_new.cuda(), slots.cuda(), case.k_pool,
                  case.v_pool, case.idx_k_pool)
    torch.cuda.synchronize()
    after = host_view(case)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    want = oracle.append_kv(before["k_pool"], before["v_pool"], before["idx_k_pool"],
                            bits(k_new), bits(v_new), bits(ik_new), slots.numpy(),
                            kv_src="bf16", kv_dtype="mxfp6", idx_dtype="bf16", k_scale=0.5,
                            v_scale=2.0)
    for name, w in zip(("k_pool", "v_pool", "idx_k_pool"), want):
        assert np.array_equal(after[name].view(np.uint8), w.view(np.uint8)), name
