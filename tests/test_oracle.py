"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed independently of its
code: exact format definitions checked against torch's own casts, planted
scores with hand-derived selections, pure-Python brute force on tiny inputs,
dense attention from ``torch.nn.functional.scaled_dot_product_attention`` in
float64, closed forms, invariances and the log-sum-exp merge identity.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import generate, host_view

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoding

def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero survives
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_fp8_table_matches_torch_all_codes():
    tab = oracle.fp8_e4m3fn_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])


def test_fp8_table_hand_values():
    tab = oracle.fp8_e4m3fn_table()
    assert tab[0x00] == 0.0 and math.copysign(1, tab[0x80]) == -1
    assert tab[0x38] == 1.0 and tab[0xB8] == -1.0
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x01] == 2.0 ** -9          # smallest subnormal
    assert tab[0x08] == 2.0 ** -6          # smallest normal
    assert tab[0x07] == 7 * 2.0 ** -9      # largest subnormal
    # every finite code is exact in bf16: round trip through bf16 bits
    fin = tab[np.isfinite(tab)]
    as_bf16 = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, fin)


def test_fp8_scale_applied():
    codes = np.array([0x38, 0x40, 0xC8], dtype=np.uint8)
    v = oracle.decode(codes, "fp8", 1.0 / 16)
    assert list(v) == [1.0 / 16, 2.0 / 16, -4.0 / 16]


# ------------------------------------------------------- planted selection

def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _planted_inputs(case, Di=16, D=16, seed=0):
    """Build a one-sequence decode input whose block scores are the planted ones."""
    rng = np.random.default_rng(seed)
    nb, tail = case["nb"], case["tail"]
    scores = [(-0.0 if s == "-0" else float(s)) for s in case["scores"]]
    L = (nb - 1) * 128 + tail
    P = nb + 3
    perm = rng.permutation(P)
    bt = perm[:nb].astype(np.int32)[None, :]
    ik = rng.standard_normal((P, 1, 128, Di)).astype(np.float32)
    ik[:, :, :, 0] = -1000.0
    for j in range(nb):
        valid = 128 if j < nb - 1 else tail
        t = (37 * j + 11) % valid
        ik[bt[0, j], 0, t, 0] = scores[j]
    if "decoy" in case and tail < 128:
        ik[bt[0, nb - 1], 0, tail:, 0] = case["decoy"]
    iq = np.zeros((1, 1, Di), dtype=np.float32)
    iq[0, 0, 0] = 1.0
    kv = rng.standard_normal((P, 1, 128, D)).astype(np.float32)
    return dict(
        q=_bf16_bits(rng.standard_normal((1, 2, D))), idx_q=_bf16_bits(iq),
        k_pool=_bf16_bits(kv), v_pool=_bf16_bits(kv[::-1].copy()),
        idx_k_pool=_bf16_bits(ik), block_table=bt,
        seq_lens=np.array([L], dtype=np.int32), cu_seqlens_q=None,
        q_dtype="bf16", kv_dtype="bf16", idx_dtype="bf16",
        topk=case["topk"], init=case["init"], local=case["local"],
        Hq=2, Hkv=1, Hidx=1), scores


def _golden_cases():
    with open(os.path.join(GOLDEN, "planted_selection.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_planted_scores_and_selection(case):
    inp, planted = _planted_inputs(case)
    sc = oracle.block_scores(inp)
    nb = case["nb"]
    got = sc[0, 0, :nb]
    assert all(g == p for g, p in zip(got, planted)), (got, planted)
    assert np.all(np.isneginf(sc[0, 0, nb:]))
    sel, cnt = oracle.select(inp, sc)
    assert list(sel[0, 0, : cnt[0, 0]]) == case["expected"]
    assert np.all(sel[0, 0, cnt[0, 0]:] == -1)


# ---------------------------------------------------- brute force, tiny

def _tiny_case(seed, B=2, lens=(300, 77), Hq=4, Hkv=2, Hidx=1, D=8, Di=8, topk=2,
               init=1, local=1, kv="bf16", prefill_new=None, idx_value=False,
               score_type="max"):
    spec = dict(kind="decode", B=B, seq_lens=list(lens), Hq=Hq, Hkv=Hkv, Hidx=Hidx,
                D=D, Di=Di, topk=topk, init=init, local=local, q="bf16", kv=kv,
                idx="bf16", k_scale=0.5 if kv == "fp8" else 1.0,
                v_scale=0.25 if kv == "fp8" else 1.0, idx_value=idx_value,
                score_type=score_type)
    if prefill_new is not None:
        spec.update(kind="prefill", n_new=list(prefill_new),
                    prefix=[L - n for L, n in zip(lens, prefill_new)])
    inp = host_view(generate(spec, seed))
    inp["_pos"] = _spec_positions(spec)
    return inp


def _spec_positions(spec):
    """(sequence, position) of every query row, written from the case's own
    description and not from the oracle: decode queries sit at seq_len - 1;
    a prefill chunk's i-th new token sits at prefix + i (the new tokens follow
    the prefix the sglang page hands over beside cu_seqlens in forward_extend)."""
    if spec["kind"] == "decode":
        return [(b, L - 1) for b, L in enumerate(spec["seq_lens"])]
    return [(b, spec["prefix"][b] + i) for b in range(spec["B"]) for i in range(spec["n_new"][b])]


def _py_value(raw, dtype, scale=1.0):
    if dtype == "bf16":
        return torch.tensor(int(np.int16(raw.view(np.int16)))).to(torch.int16).view(
            torch.bfloat16).double().item()
    if dtype == "fp8":
        return torch.tensor(int(raw), dtype=torch.uint8).view(
            torch.float8_e4m3fn).double().item() * scale
    return float(raw)


class _RowCache:
    """Stored rows decoded one scalar at a time (``_py_value``), each once."""

    def __init__(self, pool, dtype, scale=1.0):
        self.pool, self.dtype, self.scale, self.rows = pool, dtype, scale, {}

    def __call__(self, page, h, s):
        key = (page, h, s)
        if key not in self.rows:
            self.rows[key] = [_py_value(x, self.dtype, self.scale) for x in self.pool[page, h, s]]
        return self.rows[key]


def _py_scores(inp):
    """Block scores with explicit loops over blocks and tokens; query
    positions from the case description (``_spec_positions``)."""
    out = {}
    ikc = _RowCache(inp["idx_k_pool"], "bf16")
    for t, (b, p) in enumerate(inp["_pos"]):
        for h in range(inp["Hidx"]):
            iq = [_py_value(x, "bf16") for x in inp["idx_q"][t, h]]
            row = []
            j = 0
            while j * 128 <= p:
                page = int(inp["block_table"][b, j])
                best = -math.inf
                for s in range(128):
                    if j * 128 + s > p:
                        break
                    ik = ikc(page, h, s)
                    best = max(best, sum(a * c for a, c in zip(iq, ik)))
                row.append(best)
                j += 1
            out[(t, h)] = row
    return out


@pytest.mark.parametrize("seed", [1, 2])
def test_scores_brute_force(seed):
    inp = _tiny_case(seed)
    sc = oracle.block_scores(inp)
    ref = _py_scores(inp)
    for (t, h), row in ref.items():
        assert np.allclose(sc[t, h, : len(row)], row, rtol=1e-13, atol=1e-13)
        assert np.all(np.isneginf(sc[t, h, len(row):]))


def test_batched_scores_equal_per_query_definition():
    inp = _tiny_case(5, lens=(700, 260), prefill_new=(40, 260))
    sc = oracle.block_scores(inp)
    for t, (b, p) in enumerate(inp["_pos"]):
        for h in range(inp["Hidx"]):
            ik = oracle.decode(inp["idx_k_pool"][inp["block_table"][b, : (p // 128 + 1)], h]
                               .reshape(-1, inp["idx_k_pool"].shape[-1]), "bf16")
            one = oracle.block_scores_for_query(oracle.decode(inp["idx_q"][t, h], "bf16"), ik, p)
            assert np.array_equal(sc[t, h, : len(one)], one)


@pytest.mark.parametrize("nb,init,local,topk", [(7, 1, 2, 2), (9, 0, 0, 3), (8, 2, 1, 4),
                                                (6, 1, 2, 8), (10, 0, 3, 1)])
def test_selection_brute_force(nb, init, local, topk):
    rng = np.random.default_rng(nb * 100 + topk)
    for trial in range(30):
        # integer scores to force many exact ties
        s = rng.integers(-3, 4, size=nb).astype(np.float64)
        S = oracle.select_for_query(s, nb, topk, init, local)
        F = set(range(min(init, nb))) | set(range(max(0, nb - local), nb))
        C = [j for j in range(nb) if j not in F]
        k = min(topk, len(C))

        def beats(a, b):  # a ranks before b
            return s[a] > s[b] or (s[a] == s[b] and a < b)

        winners = [set(T) for T in itertools.combinations(C, k)
                   if all(beats(a, b) for a in T for b in C if b not in T)]
        assert len(winners) == 1
        assert S == sorted(F | winners[0])
        assert len(S) == min(nb, len(F) + topk)


def _py_attend(inp, sel, cnt, scale):
    """Attention with explicit loops over heads and tokens; query positions
    from the case description."""
    Hq, Hkv, Hidx = inp["Hq"], inp["Hkv"], inp["Hidx"]
    G = Hq // Hkv
    outs = {}
    kc = _RowCache(inp["k_pool"], inp["kv_dtype"], inp["k_scale"])
    vc = _RowCache(inp["v_pool"], inp["kv_dtype"], inp["v_scale"])
    for t, (b, p) in enumerate(inp["_pos"]):
        for hq in range(Hq):
            g = hq // G
            h = g // (Hkv // Hidx)
            q = [_py_value(x, inp["q_dtype"]) for x in inp["q"][t, hq]]
            zs, vs = [], []
            for j in sel[t, h, : cnt[t, h]]:
                page = int(inp["block_table"][b, j])
                for s in range(128):
                    if j * 128 + s > p:
                        break
                    k = kc(page, g, s)
                    v = vc(page, g, s)
                    zs.append(scale * sum(a * c for a, c in zip(q, k)))
                    vs.append(v)
            m = max(zs)
            e = [math.exp(z - m) for z in zs]
            tot = sum(e)
            o = [sum(e[i] * vs[i][d] for i in range(len(e))) / tot for d in range(len(q))]
            outs[(t, hq)] = (o, m + math.log(tot))
    return outs


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attention_brute_force(kv):
    inp = _tiny_case(3, lens=(300, 130), Hq=4, Hkv=2, Hidx=2, kv=kv)
    res = oracle.sparse_attention(inp)
    ref = _py_attend(inp, res["sel"], res["count"], 1.0 / math.sqrt(8))
    for (t, hq), (o, l) in ref.items():
        assert np.allclose(res["out"][t, hq], o, rtol=1e-12, atol=1e-12)
        assert abs(res["lse"][t, hq] - l) < 1e-12


# ------------------------------------------- prefill query positions

def _prefill_tiny(seed=5, lens=(700, 260), new=(40, 100), **kw):
    return _tiny_case(seed, lens=lens, prefill_new=new, **kw)


def _check_prefill_scores_brute_force():
    inp = _prefill_tiny(Hidx=2, Hkv=2)
    sc = oracle.block_scores(inp)
    ref = _py_scores(inp)
    for (t, h), row in ref.items():
        assert np.allclose(sc[t, h, : len(row)], row, rtol=1e-13, atol=1e-13), (t, h)
        assert np.all(np.isneginf(sc[t, h, len(row):])), (t, h)


def _check_prefill_attention_brute_force():
    inp = _prefill_tiny(Hq=2, Hkv=1, Hidx=1, topk=1)
    res = oracle.sparse_attention(inp)
    ref = _py_attend(inp, res["sel"], res["count"], 1.0 / math.sqrt(8))
    for (t, hq), (o, l) in ref.items():
        assert np.allclose(res["out"][t, hq], o, rtol=1e-12, atol=1e-12), (t, hq)
        assert abs(res["lse"][t, hq] - l) < 1e-12, (t, hq)


def _check_prefill_equals_full_sequence_causal_sdpa():
    """A chunk of the sequence's last n tokens, every block selected, equals
    the last n rows of plain causal attention over the whole sequence
    (torch SDPA, is_causal=True on the square L x L problem, float64), whose
    other query rows are filler: no position enters this check."""
    lens, new = (600, 300), (600, 77)
    inp = _prefill_tiny(seed=13, lens=lens, new=new, Hq=4, Hkv=2, Hidx=1, D=16, Di=8, topk=8)
    res = oracle.sparse_attention(inp)
    q = torch.from_numpy(oracle.decode(inp["q"], "bf16"))
    rng = torch.Generator().manual_seed(4)
    row = 0
    for b, (L, n) in enumerate(zip(lens, new)):
        nbk = (L + 127) // 128
        pages = inp["block_table"][b, :nbk].astype(np.int64)
        k = torch.from_numpy(oracle.decode(inp["k_pool"][pages], "bf16"))
        v = torch.from_numpy(oracle.decode(inp["v_pool"][pages], "bf16"))
        k = k.permute(1, 0, 2, 3).reshape(2, nbk * 128, 16)[:, :L].repeat_interleave(2, dim=0)
        v = v.permute(1, 0, 2, 3).reshape(2, nbk * 128, 16)[:, :L].repeat_interleave(2, dim=0)
        qf = torch.randn(4, L, 16, generator=rng, dtype=torch.float64)
        qf[:, L - n:] = q[row:row + n].permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(qf, k, v, is_causal=True)
        assert np.allclose(res["out"][row:row + n], o[:, L - n:].permute(1, 0, 2).numpy(),
                           rtol=1e-11, atol=1e-12), b
        row += n


def test_prefill_scores_brute_force():
    """Per-query causal block maxima of a prefill chunk (two sequences, one
    partly new, one all new) by explicit loops at the positions prefix + i."""
    _check_prefill_scores_brute_force()


def test_prefill_attention_brute_force():
    _check_prefill_attention_brute_force()


def test_prefill_equals_full_sequence_causal_sdpa():
    _check_prefill_equals_full_sequence_causal_sdpa()


def test_prefill_positions_golden():
    """Hand-written positions for a ragged cu_seqlens_q with an empty chunk
    (tests/golden/prefill_positions.json), and the blocks each query scores."""
    with open(os.path.join(GOLDEN, "prefill_positions.json")) as f:
        g = json.load(f)
    sl, cu = np.array(g["seq_lens"]), np.array(g["cu_seqlens_q"])
    assert oracle.query_positions(sl, cu) == [tuple(x) for x in g["expected"]]
    n_new = [int(cu[b + 1] - cu[b]) for b in range(len(sl))]
    inp = _tiny_case(3, B=len(sl), lens=tuple(int(x) for x in sl), prefill_new=n_new, topk=2)
    sc = oracle.block_scores(inp)
    for t, nb in enumerate(g["nb"]):
        assert np.isfinite(sc[t, 0, :nb]).all() and np.isneginf(sc[t, 0, nb:]).all(), t


@pytest.mark.parametrize("shift", [-1, 1])
def test_position_pins_catch_an_off_by_one(monkeypatch, shift):
    """A prefill position map off by one (p = L - n + i +- 1), planted in the
    oracle on the CPU, fails every prefill position pin above."""
    good = oracle.msa_oracle.query_positions

    def shifted(seq_lens, cu_seqlens_q, positions=None):
        pos = good(seq_lens, cu_seqlens_q, positions)
        if cu_seqlens_q is None or positions is not None:
            return pos
        return [(b, p + shift) for b, p in pos]

    monkeypatch.setattr(oracle.msa_oracle, "query_positions", shifted)
    for check in (_check_prefill_scores_brute_force, _check_prefill_attention_brute_force,
                  _check_prefill_equals_full_sequence_causal_sdpa):
        with pytest.raises((AssertionError, IndexError, ValueError)):
            check()


# ------------------------------------------ dense equivalence (library pin)

def _dense_sdpa(inp, scale=None):
    """All visible tokens, via torch SDPA in float64 with an explicit causal
    mask at the query positions of the case description."""
    q = torch.from_numpy(oracle.decode(inp["q"], inp["q_dtype"]))
    T, Hq, D = q.shape
    G = Hq // inp["Hkv"]
    out = torch.zeros(T, Hq, D, dtype=torch.float64)
    pos = inp["_pos"]
    for b in range(len(inp["seq_lens"])):
        L = int(inp["seq_lens"][b])
        toks = [t for t, (bb, _) in enumerate(pos) if bb == b]
        if L == 0 or not toks:
            continue
        nbk = (L + 127) // 128
        pages = inp["block_table"][b, :nbk].astype(np.int64)
        k = oracle.decode(inp["k_pool"][pages], inp["kv_dtype"], inp["k_scale"])
        v = oracle.decode(inp["v_pool"][pages], inp["kv_dtype"], inp["v_scale"])
        k = torch.from_numpy(k).permute(1, 0, 2, 3).reshape(inp["Hkv"], nbk * 128, D)[:, :L]
        v = torch.from_numpy(v).permute(1, 0, 2, 3).reshape(inp["Hkv"], nbk * 128, D)[:, :L]
        k = k.repeat_interleave(G, dim=0)
        v = v.repeat_interleave(G, dim=0)
        qs = q[toks].permute(1, 0, 2)                                  # [Hq, n, D]
        ps = torch.tensor([pos[t][1] for t in toks])
        mask = torch.arange(L)[None, :] <= ps[:, None]                 # [n, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            qs, k, v, attn_mask=mask, scale=scale)
        out[toks] = o.permute(1, 0, 2)
    return out.numpy()


@pytest.mark.parametrize("kv,prefill", [("bf16", None), ("f32", None), ("fp8", None),
                                        ("bf16", (100, 256))])
def test_full_coverage_equals_dense_attention(kv, prefill):
    # topk + |F| >= nb for every query: selection covers all visible blocks
    inp = _tiny_case(11, lens=(1000, 600), Hq=6, Hkv=3, Hidx=1, D=16, Di=8, topk=8,
                     kv=kv, prefill_new=prefill)
    res = oracle.sparse_attention(inp)
    dense = _dense_sdpa(inp)
    assert np.allclose(res["out"], dense, rtol=1e-11, atol=1e-12)


def test_dense_equivalence_with_explicit_scale():
    inp = _tiny_case(12, lens=(500, 900), Hq=4, Hkv=2, Hidx=2, D=16, Di=8, topk=8)
    res = oracle.sparse_attention(inp, scale=0.37)
    dense = _dense_sdpa(inp, scale=0.37)
    assert np.allclose(res["out"], dense, rtol=1e-11, atol=1e-12)


def _compacted(inp, sel, cnt):
    """The sglang page's dense-sparse form: a page table holding only each
    sequence's selected blocks, in order, and the length that covers them
    (every selected block is full but the last, the query's own)."""
    B, K = sel.shape[0], sel.shape[2]
    bt = np.full((B, K), -1, dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        c = int(cnt[b, 0])
        blocks = sel[b, 0, :c]
        bt[b, :c] = inp["block_table"][b, blocks]
        L = int(inp["seq_lens"][b])
        nb = (L + 127) // 128
        assert blocks[-1] == nb - 1
        lens[b] = 128 * (c - 1) + (L - 128 * (nb - 1))
    return dict(inp, block_table=bt, seq_lens=lens, _pos=[(b, int(n) - 1) for b, n in enumerate(lens)])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sparse_equals_dense_over_compacted_table(kv):
    """Sparse decode over the selection equals dense causal attention (torch
    SDPA, float64) over a page table compacted to the selected blocks, the
    equivalence the sglang page's dense-sparse decode relies on."""
    inp = _tiny_case(21, lens=(1500, 700, 129), B=3, Hq=4, Hkv=2, Hidx=1, D=16, Di=8, topk=2,
                     init=1, local=2, kv=kv)
    res = oracle.sparse_attention(inp)
    assert (res["count"] < (np.asarray(inp["seq_lens"]) + 127) // 128).any()  # really sparse
    dense = _dense_sdpa(_compacted(inp, res["sel"], res["count"]))
    assert np.allclose(res["out"], dense, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------- invariances

def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((8, 32))
    k = rng.standard_normal((300, 32)) * 4
    v = rng.standard_normal((300, 32))
    _, _, w = oracle.softmax_attention(q, k, v, 1 / math.sqrt(32), return_weights=True)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
    assert np.all(w >= 0)


def test_page_permutation_invariance():
    inp = _tiny_case(21, lens=(1500, 900), Hq=4, Hkv=2, Hidx=2, D=16, Di=16, topk=3)
    res = oracle.sparse_attention(inp)
    P = inp["k_pool"].shape[0]
    perm = np.random.default_rng(3).permutation(P)
    inp2 = dict(inp)
    for key in ("k_pool", "v_pool", "idx_k_pool"):
        new = np.empty_like(inp[key])
        new[perm] = inp[key]
        inp2[key] = new
    bt = inp["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    inp2["block_table"] = bt
    res2 = oracle.sparse_attention(inp2)
    for key in ("sel", "count", "out", "lse"):
        assert np.array_equal(res[key], res2[key]), key
    assert np.array_equal(res["scores"], res2["scores"])


# ------------------------------------------------------------ closed forms

def test_constant_values_give_constant_output():
    inp = _tiny_case(31, lens=(800, 260), topk=2)
    inp["v_pool"] = np.full_like(inp["v_pool"], _bf16_bits([0.75])[0])
    res = oracle.sparse_attention(inp)
    assert np.all(np.abs(res["out"] - 0.75) < 1e-14)


def test_zero_query_gives_mean_of_selected_values():
    inp = _tiny_case(32, lens=(800, 260), Hq=2, Hkv=1, Hidx=1, topk=2)
    inp["q"] = np.zeros_like(inp["q"])
    res = oracle.sparse_attention(inp)
    for t, (b, p) in enumerate(inp["_pos"]):
        S = res["sel"][t, 0, : res["count"][t, 0]]
        rows = []
        for j in S:
            page = inp["block_table"][b, j]
            n = min(128, p + 1 - 128 * j)
            rows.append(oracle.decode(inp["v_pool"][page, 0, :n], "bf16"))
        mean = np.concatenate(rows).mean(axis=0)
        assert np.allclose(res["out"][t, 0], mean, rtol=1e-13, atol=1e-14)
        # z = 0 everywhere: lse = log(number of visible selected tokens)
        assert abs(res["lse"][t, 0] - math.log(sum(r.shape[0] for r in rows))) < 1e-13


def test_single_token_sequence_returns_its_value():
    inp = _tiny_case(33, lens=(1, 1), topk=2)
    res = oracle.sparse_attention(inp)
    G = inp["Hq"] // inp["Hkv"]
    for b in range(2):
        page = inp["block_table"][b, 0]
        for hq in range(inp["Hq"]):
            v0 = oracle.decode(inp["v_pool"][page, hq // G, 0], "bf16")
            assert np.array_equal(res["out"][b, hq], v0)


def test_empty_sequence_gives_zero_output():
    inp = _tiny_case(34, lens=(0, 300), topk=2)
    res = oracle.sparse_attention(inp)
    assert res["count"][0].sum() == 0 and np.all(res["sel"][0] == -1)
    assert np.all(res["out"][0] == 0) and np.all(np.isneginf(res["lse"][0]))
    assert res["count"][1, 0] == 3          # nb = 3 blocks, all selected


def test_lse_combine_equals_unsplit():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((8, 64))
    k = rng.standard_normal((700, 64))
    v = rng.standard_normal((700, 64))
    full_o, full_l = oracle.softmax_attention(q, k, v, 0.125)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 700), size=rng.integers(1, 9), replace=False))
        parts = np.split(np.arange(700), cuts)
        os_, ls_ = zip(*[oracle.softmax_attention(q, k[ix], v[ix], 0.125) for ix in parts])
        o, l = oracle.lse_combine(np.stack(os_), np.stack(ls_))
        assert np.allclose(o, full_o, rtol=1e-13, atol=1e-13)
        assert np.allclose(l, full_l, rtol=1e-13, atol=1e-13)
    # an empty part (lse = -inf, o = 0) changes nothing
    o, l = oracle.lse_combine(np.stack([full_o, np.zeros_like(full_o)]),
                              np.stack([full_l, np.full_like(full_l, -np.inf)]))
    assert np.allclose(o, full_o, rtol=1e-15) and np.allclose(l, full_l, rtol=1e-15)


def test_selection_structure_on_random_case():
    inp = _tiny_case(41, lens=(3000, 2000), Hq=4, Hkv=2, Hidx=2, D=8, Di=8, topk=3,
                     init=1, local=2)
    res = oracle.sparse_attention(inp)
    for t, (b, p) in enumerate(inp["_pos"]):
        nb = p // 128 + 1
        for h in range(2):
            S = list(res["sel"][t, h, : res["count"][t, h]])
            assert S == sorted(set(S))
            F = oracle.forced_blocks(nb, 1, 2)
            assert set(F) <= set(S)
            assert len(S) == min(nb, len(F) + 3)


# ---------------------------------------------------------------- paged append

def test_fp8_encode_matches_torch_cast():
    """The oracle's e4m3fn encoder (nearest code, ties to even, written from the
    format) against torch's float32 -> float8_e4m3fn cast on the CPU, over
    normals, subnormals, values past the largest finite one (clamped first:
    the stored code saturates) and exact midpoints between neighbouring codes."""
    rng = np.random.default_rng(7)
    n = 30000
    y = (rng.standard_normal(n) * np.exp(rng.uniform(-14.0, 8.0, n))).astype(np.float32)
    tab = oracle.fp8_e4m3fn_table()
    fin = tab[:0x7F]
    mids = ((fin[:-1] + fin[1:]) / 2.0).astype(np.float32)   # exact in float32
    y = np.concatenate([y, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0, 1e30, -1e30])])
    mine = oracle.fp8_e4m3fn_encode(y)
    ref = torch.from_numpy(np.clip(y, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(mine, ref.numpy())


def test_fp8_encode_round_trip_ties_and_saturation():
    tab = oracle.fp8_e4m3fn_table()
    codes = np.array([c for c in range(256) if not math.isnan(tab[c])], dtype=np.int64)
    # every finite code is its own nearest value (the -0 code keeps its sign)
    assert np.array_equal(oracle.fp8_e4m3fn_encode(tab[codes].astype(np.float32)), codes)
    # a value halfway between two neighbouring codes takes the even one
    for c in range(0x7E):
        mid = np.float32((tab[c] + tab[c + 1]) / 2.0)
        want = c if c % 2 == 0 else c + 1
        assert oracle.fp8_e4m3fn_encode(np.float32([mid]))[0] == want
        assert oracle.fp8_e4m3fn_encode(np.float32([-mid]))[0] == want | 0x80
    # just above / below a midpoint goes to the nearer code
    m = np.float32((tab[0x31] + tab[0x32]) / 2.0)
    assert oracle.fp8_e4m3fn_encode(np.nextafter(m, np.float32(10.0), dtype=np.float32)[None])[0] == 0x32
    assert oracle.fp8_e4m3fn_encode(np.nextafter(m, np.float32(0.0), dtype=np.float32)[None])[0] == 0x31
    # saturation at the largest finite magnitude, 448 = 0x7E
    assert list(oracle.fp8_e4m3fn_encode(np.float32([500.0, 1e38, -465.0]))) == [0x7E, 0x7E, 0xFE]
    # a negative value below half the smallest subnormal rounds to -0
    assert oracle.fp8_e4m3fn_encode(np.float32([-2.0 ** -11]))[0] == 0x80
    assert oracle.fp8_e4m3fn_encode(np.float32([2.0 ** -11]))[0] == 0x00


@pytest.mark.parametrize("kv", ["bf16", "f32", "fp8", "fp8_e5m2"])
def test_append_kv_oracle(kv):
    """append_kv writes token t's rows at page slot//128, offset slot%128 of
    every head, leaves all other rows untouched and skips slots outside the
    pool; an fp8 pool holds the code of x / scale (bf16 x, float32 division),
    which decodes back to x when x / scale is an e4m3 value."""
    rng = np.random.default_rng(11)
    P, Hkv, Hidx, D, Di, T = 5, 2, 1, 8, 4, 7
    src = "f32" if kv == "f32" else "bf16"

    def rand_src(shape, dt):
        x = rng.standard_normal(shape).astype(np.float32)
        return x if dt == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)

    pool_dt = {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8, "fp8_e5m2": np.uint8}[kv]
    k_pool = rng.integers(0, 2 ** 7, (P, Hkv, 128, D)).astype(pool_dt)
    v_pool = rng.integers(0, 2 ** 7, (P, Hkv, 128, D)).astype(pool_dt)
    ik_pool = rand_src((P, Hidx, 128, Di), "bf16")
    k_new, v_new = rand_src((T, Hkv, D), src), rand_src((T, Hkv, D), src)
    ik_new = rand_src((T, Hidx, Di), "bf16")
    slots = np.array([3, 128 * 2 + 127, -1, 128 * 4, P * 128, 77, 128 + 5], dtype=np.int64)
    ks, vs = 0.25, 0.125
    k2, v2, ik2 = oracle.append_kv(k_pool, v_pool, ik_pool, k_new, v_new, ik_new, slots,
                                   kv_src=src, kv_dtype=kv, idx_dtype="bf16", k_scale=ks,
                                   v_scale=vs)
    written = np.zeros((P, 128), dtype=bool)
    for t, s in enumerate(slots):
        if 0 <= s < P * 128:
            page, off = divmod(int(s), 128)
            written[page, off] = True
            assert np.array_equal(ik2[page, :, off], ik_new[t])
            if kv.startswith("fp8"):
                tdt, top = ((torch.float8_e4m3fn, 448.0) if kv == "fp8"
                            else (torch.float8_e5m2, 57344.0))
                for pool, new, sc in ((k2, k_new, ks), (v2, v_new, vs)):
                    want = torch.from_numpy(
                        (oracle.decode(new[t], "bf16").astype(np.float32) / np.float32(sc))
                        .clip(-top, top)).to(tdt).view(torch.uint8).numpy()
                    assert np.array_equal(pool[page, :, off], want)
            else:
                assert np.array_equal(k2[page, :, off], k_new[t])
                assert np.array_equal(v2[page, :, off], v_new[t])
    for old, new in ((k_pool, k2), (v_pool, v2), (ik_pool, ik2)):
        assert np.array_equal(old.transpose(0, 2, 1, 3)[~written], new.transpose(0, 2, 1, 3)[~written])
    # e4m3 values times a power-of-two scale come back exactly
    x = oracle.fp8_e4m3fn_table()[[0x01, 0x22, 0x38, 0x5C, 0xB3, 0xFE]].astype(np.float32) / 16
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.decode(oracle.store_values(xb, "bf16", "fp8", 1 / 16), "fp8", 1 / 16), x)


def test_fp8_e5m2_table_matches_torch_all_codes():
    """The E5M2 table (from the format definition) against torch's
    float8_e5m2 -> float32 cast of all 256 codes, NaN codes included."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float32).double().numpy()
    mine = oracle.fp8_e5m2_table()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])
    # hand values: 1.0, the largest finite, the smallest subnormal, infinities
    assert mine[0x3C] == 1.0 and mine[0x7B] == 57344.0 and mine[0x01] == 2.0 ** -16
    assert mine[0x7C] == math.inf and mine[0xFC] == -math.inf


def test_fp8_e5m2_encode_matches_torch_cast():
    rng = np.random.default_rng(9)
    n = 30000
    y = (rng.standard_normal(n) * np.exp(rng.uniform(-20.0, 13.0, n))).astype(np.float32)
    tab = oracle.fp8_e5m2_table()
    fin = tab[:0x7C]
    mids = ((fin[:-1] + fin[1:]) / 2.0).astype(np.float32)
    y = np.concatenate([y, mids, -mids, np.float32([0.0, -0.0, 57344.0, 1e30, -1e30])])
    mine = oracle.fp8_e5m2_encode(y)
    ref = torch.from_numpy(np.clip(y, -57344.0, 57344.0)).to(torch.float8_e5m2).view(torch.uint8)
    assert np.array_equal(mine, ref.numpy())
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], dtype=np.int64)
    assert np.array_equal(oracle.fp8_e5m2_encode(tab[codes].astype(np.float32)), codes)


@pytest.mark.parametrize("nb,init,local,topk", [(7, 1, 2, 4), (9, 0, 0, 3), (8, 2, 1, 4),
                                                (6, 1, 2, 8), (10, 2, 3, 4), (12, 3, 3, 4)])
def test_selection_forced_in_budget_brute_force(nb, init, local, topk):
    """The budget variant: S holds every forced block and the best
    max(topk - |F|, 0) others, checked against every subset of that size;
    |S| = min(nb, max(topk, |F|))."""
    rng = np.random.default_rng(nb * 31 + topk)
    for trial in range(30):
        s = rng.integers(-3, 4, size=nb).astype(np.float64)
        S = oracle.select_for_query(s, nb, topk, init, local, forced_in_budget=True)
        F = set(range(min(init, nb))) | set(range(max(0, nb - local), nb))
        C = [j for j in range(nb) if j not in F]
        k = min(max(topk - len(F), 0), len(C))

        def beats(a, b):
            return s[a] > s[b] or (s[a] == s[b] and a < b)

        winners = [set(T) for T in itertools.combinations(C, k)
                   if all(beats(a, b) for a in T for b in C if b not in T)]
        assert len(winners) == 1
        assert S == sorted(F | winners[0])
        assert len(S) == min(nb, max(topk, len(F)))


# ------------------------------------------------------ index-value branch

def _py_index_value(inp, scale):
    """Index-value attention with explicit loops over heads and tokens, at the
    positions of the case description."""
    ikc = _RowCache(inp["idx_k_pool"], "bf16")
    ivc = _RowCache(inp["idx_v_pool"], "bf16")
    outs = {}
    for t, (b, p) in enumerate(inp["_pos"]):
        for h in range(inp["Hidx"]):
            q = [_py_value(x, "bf16") for x in inp["idx_q"][t, h]]
            zs, vs = [], []
            for tok in range(p + 1):
                page = int(inp["block_table"][b, tok // 128])
                k = ikc(page, h, tok % 128)
                zs.append(scale * sum(a * c for a, c in zip(q, k)))
                vs.append(ivc(page, h, tok % 128))
            m = max(zs)
            e = [math.exp(z - m) for z in zs]
            tot = sum(e)
            outs[(t, h)] = ([sum(e[i] * vs[i][d] for i in range(len(e))) / tot
                             for d in range(len(q))], m + math.log(tot))
    return outs


@pytest.mark.parametrize("prefill", [None, (40, 100)])
def test_index_value_brute_force(prefill):
    inp = _tiny_case(51, lens=(700, 260), Hq=4, Hkv=2, Hidx=2, prefill_new=prefill,
                     idx_value=True)
    out, lse = oracle.index_value_attention(inp)
    ref = _py_index_value(inp, 1.0 / math.sqrt(8))
    for (t, h), (o, l) in ref.items():
        assert np.allclose(out[t, h], o, rtol=1e-12, atol=1e-12), (t, h)
        assert abs(lse[t, h] - l) < 1e-12, (t, h)


def test_index_value_equals_causal_sdpa():
    """Every index head of a chunk of the last n tokens (and of decode) against
    torch SDPA, is_causal=True over the whole sequence in float64, whose other
    query rows are filler: no position enters the check."""
    lens, new = (900, 300), (900, 64)
    inp = _tiny_case(52, lens=lens, Hq=4, Hkv=2, Hidx=2, Di=16, prefill_new=new,
                     idx_value=True)
    out, _ = oracle.index_value_attention(inp)
    iq = torch.from_numpy(oracle.decode(inp["idx_q"], "bf16"))
    rng = torch.Generator().manual_seed(5)
    row = 0
    for b, (L, n) in enumerate(zip(lens, new)):
        nbk = (L + 127) // 128
        pages = inp["block_table"][b, :nbk].astype(np.int64)
        k = torch.from_numpy(oracle.decode(inp["idx_k_pool"][pages], "bf16"))
        v = torch.from_numpy(oracle.decode(inp["idx_v_pool"][pages], "bf16"))
        k = k.permute(1, 0, 2, 3).reshape(2, nbk * 128, 16)[:, :L]
        v = v.permute(1, 0, 2, 3).reshape(2, nbk * 128, 16)[:, :L]
        qf = torch.randn(2, L, 16, generator=rng, dtype=torch.float64)
        qf[:, L - n:] = iq[row:row + n].permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(qf, k, v, is_causal=True)
        assert np.allclose(out[row:row + n], o[:, L - n:].permute(1, 0, 2).numpy(),
                           rtol=1e-11, atol=1e-12), b
        row += n


def test_index_value_closed_forms():
    inp = _tiny_case(53, lens=(500, 1, 129), B=3, Hidx=1, idx_value=True)
    # a zero index query weighs every visible token equally
    inp["idx_q"] = np.zeros_like(inp["idx_q"])
    out, lse = oracle.index_value_attention(inp)
    for t, (b, p) in enumerate(inp["_pos"]):
        pages = inp["block_table"][b, : p // 128 + 1].astype(np.int64)
        rows = oracle.decode(inp["idx_v_pool"][pages, 0].reshape(-1, 8)[: p + 1], "bf16")
        assert np.allclose(out[t, 0], rows.mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[t, 0] - math.log(p + 1)) < 1e-13
    # a single visible token returns its value; constant values return the constant
    page = inp["block_table"][1, 0]
    assert np.array_equal(out[1, 0], oracle.decode(inp["idx_v_pool"][page, 0, 0], "bf16"))
    inp["idx_v_pool"] = np.full_like(inp["idx_v_pool"], _bf16_bits([-1.25])[0])
    out, _ = oracle.index_value_attention(inp)
    assert np.all(np.abs(out - (-1.25)) < 1e-14)


def test_index_value_empty_sequence_and_append():
    inp = _tiny_case(54, lens=(0, 300), Hidx=1, idx_value=True)
    out, lse = oracle.index_value_attention(inp)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    # the append stores index values beside the index keys
    rng = np.random.default_rng(3)
    P = 3
    pools = [rng.integers(0, 1 << 14, (P, 1, 128, 8)).astype(np.uint16) for _ in range(4)]
    new = [rng.integers(0, 1 << 14, (2, 1, 8)).astype(np.uint16) for _ in range(4)]
    res = oracle.append_kv(*pools[:3], *new[:3], np.array([130, 5]), kv_src="bf16",
                           kv_dtype="bf16", idx_dtype="bf16", idx_v_pool=pools[3],
                           idx_v_new=new[3])
    assert len(res) == 4
    assert np.array_equal(res[3][1, :, 2], new[3][0]) and np.array_equal(res[3][0, :, 5], new[3][1])


# ------------------------------------------------------------- MX-fp4 pools

def test_e2m1_table_from_the_format():
    """E2M1: the eight magnitudes the format definition gives (0, the
    subnormal 0.5, then 1 .. 6), negated by the sign bit; each is exactly an
    e4m3 value, and the e4m3 code with the same sign, exponent (rebiased from
    1 to 7) and mantissa (shifted up two bits) holds it (e4m3 table pinned
    against torch's cast above)."""
    tab = oracle.fp4_e2m1_table()
    assert list(tab[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(tab[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert math.copysign(1.0, tab[8]) == -1.0
    e4 = oracle.fp8_e4m3fn_table()
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 1:
            e4code = (s << 7) | 0x30            # 0.5 = 2^-1: e4m3 exponent field 6
        elif e == 0:
            e4code = s << 7
        else:
            e4code = (s << 7) | ((e - 1 + 7) << 3) | (m << 2)
        assert tab[c] == e4[e4code], c
    got = torch.from_numpy(tab).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, tab)


def test_e8m0_table_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = oracle.e8m0_table()
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])


def _brute_group(x, tab=None, maxv=6.0):
    """One group of 32 float32 values, brute force: the largest k with
    2^k <= max|x| (by repeated doubling), scale 2^(k-2) (clamped to the E8M0
    range; 2 is the largest exponent of E2M1 and of E2M3 alike), and per
    element the code nearest to x / scale among all of the element format's
    codes (E2M1 by default; the upper half of the codes are the negatives),
    ties to the even code."""
    amax = max(abs(float(v)) for v in x)
    if amax == 0:
        sc = 0
    else:
        k = 0
        while 2.0 ** (k + 1) <= amax:
            k += 1
        while 2.0 ** k > amax:
            k -= 1
        sc = min(max(k - 2 + 127, 0), 254)
    X = 2.0 ** (sc - 127)
    tab = oracle.fp4_e2m1_table() if tab is None else tab
    n = len(tab)
    codes = []
    for v in x:
        y = min(max(float(v) / X, -maxv), maxv)
        d = [abs(y - tab[c]) for c in range(n)]
        sign_ok = [c for c in range(n) if (c >= n // 2) == (math.copysign(1.0, y) < 0)]
        best = min(d[c] for c in sign_ok)
        cands = [c for c in sign_ok if d[c] == best]
        even = [c for c in cands if c % 2 == 0]
        codes.append((even or cands)[0])
    return sc, codes


def test_mxfp4_encoder_brute_force():
    rng = np.random.default_rng(17)
    groups = [rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** rng.integers(-6, 7))
              for _ in range(40)]
    tab = oracle.fp4_e2m1_table()
    # exact midpoints between neighbouring codes, scaled: ties to the even code
    mids = np.array([(tab[i] + tab[i + 1]) / 2 for i in range(7)] * 4 + [6.0] * 4, dtype=np.float32)
    groups.append(mids)
    groups.append(-mids)
    groups.append(np.zeros(32, dtype=np.float32))
    groups.append(np.array([7.9] + [0.01] * 31, dtype=np.float32))   # saturates at 6 * scale
    x = np.stack(groups)
    packed, sc = oracle.mxfp4_encode_rows(x)
    for gi, grp in enumerate(groups):
        want_sc, want_codes = _brute_group(grp)
        assert sc[gi, 0] == want_sc, gi
        got = [(packed[gi, i // 2] >> (4 * (i % 2))) & 0xF for i in range(32)]
        assert got == want_codes, gi


def test_mxfp4_run_layout_and_round_trip():
    """Run layout (codes of token t at bytes t * D / 2 .., element 2i in the
    low nibble; scales after all codes) and values of the form code * 2^k that
    come back exactly."""
    D = 64
    rng = np.random.default_rng(5)
    tab = oracle.fp4_e2m1_table()
    codes = rng.integers(0, 16, (128, D))
    codes[:, ::32] = 7                       # every group holds a 6: scale = its 2^k
    k = rng.integers(-4, 5, (128, D // 32))
    vals = (tab[codes] * np.repeat(2.0 ** k, 32, axis=1)).astype(np.float32)
    run = oracle.mxfp4_encode_run_rows(vals[None])[0]
    assert run.shape == (oracle.mxfp4_run_bytes(D),)
    assert run[0] & 0xF == codes[0, 0] and run[0] >> 4 == codes[0, 1]
    assert run[D // 2 * 5 + 3] >> 4 == codes[5, 7]
    assert run[128 * D // 2 + 2 * 9 + 1] == k[9, 1] + 127
    dec = oracle.mxfp4_decode_runs(run[None], D)[0]
    assert np.array_equal(dec, vals.astype(np.float64))
    # a NaN scale code decodes its group to NaN
    bad = run.copy()
    bad[128 * D // 2] = 0xFF
    dec = oracle.mxfp4_decode_runs(bad[None], D)[0]
    assert np.isnan(dec[0, :32]).all() and not np.isnan(dec[0, 32:]).any()


def test_mxfp4_synthetic_pools_follow_the_encoder():
    """The generator's MX-fp4 pools are the oracle encoder's bytes of the same
    float draws (the generator holds its own vectorised copy of the rule)."""
    from synth.inputs import _mxfp4_runs
    g = torch.Generator().manual_seed(9)
    x = torch.randn((3, 2, 128, 128), generator=g) * 1.7
    mine = _mxfp4_runs(x).numpy()
    ref = oracle.mxfp4_encode_run_rows(x.numpy())
    assert np.array_equal(mine, ref)


@pytest.mark.parametrize("prefill", [None, (100, 256)])
def test_mxfp4_attention_dense_equivalence_and_brute_force(prefill):
    inp = _tiny_case(61, lens=(1000, 600), Hq=6, Hkv=3, Hidx=1, D=64, Di=8, topk=8,
                     kv="mxfp4", prefill_new=prefill)
    res = oracle.sparse_attention(inp)
    # dense causal SDPA over the decoded pools
    q = torch.from_numpy(oracle.decode(inp["q"], "bf16"))
    for b, L in enumerate(inp["seq_lens"]):
        L = int(L)
        nbk = (L + 127) // 128
        pages = inp["block_table"][b, :nbk].astype(np.int64)
        k = torch.from_numpy(oracle.mxfp4_decode_runs(inp["k_pool"][pages], 64))
        v = torch.from_numpy(oracle.mxfp4_decode_runs(inp["v_pool"][pages], 64))
        k = k.permute(1, 0, 2, 3).reshape(3, -1, 64)[:, :L].repeat_interleave(2, dim=0)
        v = v.permute(1, 0, 2, 3).reshape(3, -1, 64)[:, :L].repeat_interleave(2, dim=0)
        toks = [t for t, (bb, _) in enumerate(inp["_pos"]) if bb == b]
        ps = torch.tensor([inp["_pos"][t][1] for t in toks])
        mask = torch.arange(L)[None, :] <= ps[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q[toks].permute(1, 0, 2), k, v,
                                                             attn_mask=mask)
        assert np.allclose(res["out"][toks], o.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_mxfp4_append_oracle():
    rng = np.random.default_rng(23)
    P, H, D, T = 3, 2, 64, 4
    run = oracle.mxfp4_run_bytes(D)
    k_pool = rng.integers(0, 256, (P, H, run)).astype(np.uint8)
    v_pool = rng.integers(0, 256, (P, H, run)).astype(np.uint8)
    ik = np.zeros((P, 1, 128, 8), dtype=np.uint16)
    xs = rng.standard_normal((T, H, D)).astype(np.float32)
    bits = (xs.view(np.uint32) >> 16).astype(np.uint16)          # bf16 by truncation
    new_ik = np.zeros((T, 1, 8), dtype=np.uint16)
    slots = np.array([5, 130, -1, 383])
    k2, v2, _ = oracle.append_kv(k_pool, v_pool, ik, bits, bits, new_ik, slots, kv_src="bf16",
                                 kv_dtype="mxfp4", idx_dtype="bf16", k_scale=0.5, v_scale=2.0)
    dk = oracle.mxfp4_decode_runs(k2, D, 0.5)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        page, off = divmod(int(s), 128)
        x = oracle.decode(bits[t], "bf16")
        err = np.abs(dk[page, :, off] - x)
        # within one E2M1 step of the group's scale (times the tensor scale)
        bound = np.repeat(np.abs(x).reshape(H, -1, 32).max(axis=-1), 32, axis=-1) / 2
        assert (err <= bound + 1e-30).all()
    changed = np.zeros((P, H, run), dtype=bool)
    for s in slots[slots >= 0]:
        page, off = divmod(int(s), 128)
        changed[page, :, off * D // 2:(off + 1) * D // 2] = True
        changed[page, :, 128 * D // 2 + off * 2:128 * D // 2 + off * 2 + 2] = True
    assert np.array_equal(k2[~changed], k_pool[~changed])


# ------------------------------------------------------------- MX-fp6 pools

def test_e2m3_table_from_the_format():
    """E2M3 (bias 1): exponent field 0 holds the subnormals m / 8, fields 1..3
    the normals 2^(e-1) (1 + m / 8) up to 7.5; the sign bit negates.  The
    normals are e4m3 values with the same mantissa bits and the exponent field
    rebiased from 1 to 7 (e4m3 table pinned against torch's cast above)."""
    tab = oracle.fp6_e2m3_table()
    want = [m / 8 for m in range(8)] + [1 + m / 8 for m in range(8)] \
        + [2 + m / 4 for m in range(8)] + [4 + m / 2 for m in range(8)]
    assert list(tab[:32]) == want
    assert tab[31] == 7.5 and tab[1] == 0.125 and tab[8] == 1.0
    assert np.array_equal(tab[32:], -tab[:32]) and math.copysign(1.0, tab[32]) < 0
    e4 = oracle.fp8_e4m3fn_table()
    for c in range(64):
        s, e, m = c >> 5, (c >> 3) & 3, c & 7
        if e:
            assert tab[c] == e4[(s << 7) | ((e + 6) << 3) | m], c


def test_fp6_bit_order():
    """Element i of a 32-group sits at bits 6 i .. 6 i + 5 of the group's 24
    bytes read as one little-endian number: checked with a literal and with
    Python's big integers on random codes."""
    assert list(oracle.fp6_pack(np.array([1, 2, 3, 4]))) == [0x81, 0x30, 0x10]
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 64, (5, 32))
    packed = oracle.fp6_pack(codes)
    assert packed.shape == (5, 24)
    for r in range(5):
        v = int.from_bytes(bytes(packed[r].tolist()), "little")
        assert [(v >> (6 * i)) & 63 for i in range(32)] == list(codes[r])
    assert np.array_equal(oracle.fp6_unpack(packed), codes)


def test_mxfp6_encoder_brute_force():
    rng = np.random.default_rng(19)
    groups = [rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** rng.integers(-6, 7))
              for _ in range(40)]
    tab = oracle.fp6_e2m3_table()
    # exact midpoints between neighbouring codes (ties to the even code), and 7.5
    mids = np.array([(tab[i] + tab[i + 1]) / 2 for i in range(31)] + [7.5], dtype=np.float32)
    groups.append(mids)
    groups.append(-mids)
    groups.append(np.zeros(32, dtype=np.float32))
    groups.append(np.array([7.9] + [0.01] * 31, dtype=np.float32))   # saturates at 7.5 * scale
    groups.append(np.array([1e-39] * 32, dtype=np.float32))          # subnormal float32 group
    x = np.stack(groups)
    packed, sc = oracle.mxfp6_encode_rows(x)
    codes = oracle.fp6_unpack(packed)
    for gi, grp in enumerate(groups):
        want_sc, want_codes = _brute_group(grp, tab, 7.5)
        assert sc[gi, 0] == want_sc, gi
        assert list(codes[gi]) == want_codes, gi


def test_mxfp6_run_layout_and_round_trip():
    """Run layout (codes of token t at bytes t * 3 D / 4 ..; scales after all
    codes) and values of the form code * 2^k that come back exactly."""
    D = 64
    rng = np.random.default_rng(6)
    tab = oracle.fp6_e2m3_table()
    codes = rng.integers(0, 64, (128, D))
    codes[:, ::32] = 31                      # every group holds a 7.5: scale = its 2^k
    k = rng.integers(-4, 5, (128, D // 32))
    vals = (tab[codes] * np.repeat(2.0 ** k, 32, axis=1)).astype(np.float32)
    run = oracle.mxfp6_encode_run_rows(vals[None])[0]
    assert run.shape == (oracle.mxfp6_run_bytes(D),) == (128 * D * 3 // 4 + 128 * D // 32,)
    assert run[0] & 0x3F == codes[0, 0] and (run[0] >> 6 | (run[1] & 0xF) << 2) == codes[0, 1]
    t0 = 5 * D * 3 // 4
    v = int.from_bytes(bytes(run[t0 + 24:t0 + 48].tolist()), "little")
    assert [(v >> (6 * i)) & 63 for i in range(32)] == list(codes[5, 32:])
    assert run[128 * D * 3 // 4 + 2 * 9 + 1] == k[9, 1] + 127
    dec = oracle.mxfp6_decode_runs(run[None], D)[0]
    assert np.array_equal(dec, np.where(codes == 32, -0.0, vals.astype(np.float64)))
    bad = run.copy()
    bad[128 * D * 3 // 4] = 0xFF
    dec = oracle.mxfp6_decode_runs(bad[None], D)[0]
    assert np.isnan(dec[0, :32]).all() and not np.isnan(dec[0, 32:]).any()


def test_mxfp6_synthetic_pools_follow_the_encoder():
    """The generator's MX-fp6 pools are the oracle encoder's bytes of the same
    float draws (the generator holds its own vectorised copy of the rule)."""
    from synth.inputs import _mxfp6_runs
    g = torch.Generator().manual_seed(10)
    x = torch.randn((3, 2, 128, 128), generator=g) * 1.7
    x[0, 0, 0, :32] = torch.tensor(np.array([(a + b) / 2 for a, b in zip(
        oracle.fp6_e2m3_table()[:31], oracle.fp6_e2m3_table()[1:32])] + [7.5], dtype=np.float32))
    mine = _mxfp6_runs(x).numpy()
    ref = oracle.mxfp6_encode_run_rows(x.numpy())
    assert np.array_equal(mine, ref)


@pytest.mark.parametrize("prefill", [None, (100, 256)])
def test_mxfp6_attention_dense_equivalence(prefill):
    inp = _tiny_case(62, lens=(1000, 600), Hq=6, Hkv=3, Hidx=1, D=64, Di=8, topk=8,
                     kv="mxfp6", prefill_new=prefill)
    res = oracle.sparse_attention(inp)
    q = torch.from_numpy(oracle.decode(inp["q"], "bf16"))
    tab = oracle.fp6_e2m3_table()
    for b, L in enumerate(inp["seq_lens"]):
        L = int(L)
        nbk = (L + 127) // 128
        pages = inp["block_table"][b, :nbk].astype(np.int64)
        kv = []
        for pool in (inp["k_pool"], inp["v_pool"]):
            # decoded here from the bit layout, independently of the oracle's reader
            run = pool[pages]                                         # [nbk, H, bytes]
            nc = 128 * 64 * 3 // 4
            grp = run[..., :nc].reshape(nbk, 3, 128, 2, 24).astype(np.uint64)
            vals = np.zeros((nbk, 3, 128, 2, 32))
            for i in range(32):
                byte, sh = divmod(6 * i, 8)
                c = grp[..., byte] >> np.uint64(sh)
                if sh > 2:
                    c = c | (grp[..., byte + 1] << np.uint64(8 - sh))
                vals[..., i] = tab[(c & np.uint64(63)).astype(np.int64)]
            sc = run[..., nc:].reshape(nbk, 3, 128, 2).astype(np.float64)
            kv.append(torch.from_numpy((vals * np.exp2(sc - 127)[..., None]).reshape(nbk, 3, 128, 64)))
        k, v = kv
        k = k.permute(1, 0, 2, 3).reshape(3, -1, 64)[:, :L].repeat_interleave(2, dim=0)
        v = v.permute(1, 0, 2, 3).reshape(3, -1, 64)[:, :L].repeat_interleave(2, dim=0)
        toks = [t for t, (bb, _) in enumerate(inp["_pos"]) if bb == b]
        ps = torch.tensor([inp["_pos"][t][1] for t in toks])
        mask = torch.arange(L)[None, :] <= ps[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q[toks].permute(1, 0, 2), k, v,
                                                             attn_mask=mask)
        assert np.allclose(res["out"][toks], o.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_mxfp6_append_oracle():
    rng = np.random.default_rng(29)
    P, H, D, T = 3, 2, 64, 4
    run = oracle.mxfp6_run_bytes(D)
    k_pool = rng.integers(0, 256, (P, H, run)).astype(np.uint8)
    v_pool = rng.integers(0, 256, (P, H, run)).astype(np.uint8)
    ik = np.zeros((P, 1, 128, 8), dtype=np.uint16)
    xs = rng.standard_normal((T, H, D)).astype(np.float32)
    bits = (xs.view(np.uint32) >> 16).astype(np.uint16)
    new_ik = np.zeros((T, 1, 8), dtype=np.uint16)
    slots = np.array([5, 130, -1, 383])
    k2, v2, _ = oracle.append_kv(k_pool, v_pool, ik, bits, bits, new_ik, slots, kv_src="bf16",
                                 kv_dtype="mxfp6", idx_dtype="bf16", k_scale=0.5, v_scale=2.0)
    dk = oracle.mxfp6_decode_runs(k2, D, 0.5)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        page, off = divmod(int(s), 128)
        x = oracle.decode(bits[t], "bf16")
        err = np.abs(dk[page, :, off] - x)
        # half a step of the top binade (a quarter of the scale), or the clamp
        # from below 8 to 7.5 scales: at most max|x| / 8 per group
        bound = np.repeat(np.abs(x).reshape(H, -1, 32).max(axis=-1), 32, axis=-1) / 8
        assert (err <= bound + 1e-30).all()
    nc = 128 * D * 3 // 4
    changed = np.zeros((P, H, run), dtype=bool)
    for s in slots[slots >= 0]:
        page, off = divmod(int(s), 128)
        changed[page, :, off * D * 3 // 4:(off + 1) * D * 3 // 4] = True
        changed[page, :, nc + off * 2:nc + off * 2 + 2] = True
    assert np.array_equal(k2[~changed], k_pool[~changed])


# -------------------------------------------------------------- score types

def _py_block_reduce(ds, score_type, Di):
    """A block's score from its visible dots, written out with the math module."""
    if score_type == "max":
        return max(ds)
    if score_type == "mean":
        return math.fsum(ds) / len(ds)
    zs = [d / math.sqrt(Di) for d in ds]
    m = max(zs)
    return m + math.log(math.fsum(math.exp(z - m) for z in zs))


@pytest.mark.parametrize("score_type", ["mean", "lse"])
@pytest.mark.parametrize("prefill", [None, (40, 100)])
def test_score_types_brute_force(score_type, prefill):
    """Mean and log-sum-exp block scores by explicit loops at the positions of
    the case description, decode and prefill, against the oracle's batched
    form and its per-query form."""
    inp = _tiny_case(71, lens=(700, 260), Hidx=2, Hkv=2, prefill_new=prefill,
                     score_type=score_type)
    sc = oracle.block_scores(inp)
    ikc = _RowCache(inp["idx_k_pool"], "bf16")
    for t, (b, p) in enumerate(inp["_pos"]):
        for h in range(2):
            iq = [_py_value(x, "bf16") for x in inp["idx_q"][t, h]]
            nb = p // 128 + 1
            for j in range(nb):
                page = int(inp["block_table"][b, j])
                ds = [sum(a * c for a, c in zip(iq, ikc(page, h, s_)))
                      for s_ in range(min(128, p + 1 - 128 * j))]
                want = _py_block_reduce(ds, score_type, 8)
                assert abs(sc[t, h, j] - want) <= 1e-12 * max(1.0, abs(want)), (t, h, j)
            assert np.all(np.isneginf(sc[t, h, nb:]))
            ik = oracle.decode(inp["idx_k_pool"][inp["block_table"][b, :nb], h].reshape(-1, 8),
                               "bf16")
            one = oracle.block_scores_for_query(oracle.decode(inp["idx_q"][t, h], "bf16"), ik, p,
                                                score_type)
            assert np.allclose(sc[t, h, :nb], one, rtol=1e-12, atol=1e-12)


def test_score_types_closed_forms():
    """Blocks whose visible index keys are all equal: mean = max = the common
    dot, and lse = dot / sqrt(Di) + log(number of visible tokens); the
    partial last block counts only its visible tokens."""
    inp = _tiny_case(72, lens=(300,), B=1, Hidx=1, Hkv=1, Hq=2)
    one = _bf16_bits([0.5])[0]
    inp["idx_k_pool"] = np.full_like(inp["idx_k_pool"], one)
    inp["idx_q"] = np.full_like(inp["idx_q"], one)
    d = 8 * 0.25                                          # Di = 8 products of 0.5 * 0.5
    for st, want in (("max", [d, d, d]), ("mean", [d, d, d]),
                     ("lse", [d / math.sqrt(8) + math.log(n) for n in (128, 128, 44)])):
        sc = oracle.block_scores(dict(inp, score_type=st))
        assert np.allclose(sc[0, 0, :3], want, rtol=1e-14, atol=1e-14), st
