"""GPU parity of the index-value branch (idx_out: per index head, softmax
attention of the index query over the index keys and values of every visible
token) against the fp64 oracle, through the C ABI: decode (fused into the
index scan), chunked prefill (long and short chunks) and the append of index
values.  The branch leaves the attention output, lse and selection bit for
bit as they are with it off."""

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


def _dec(B, lens, Hq=16, Hkv=2, Hidx=2, Di=128, topk=8, q="bf16", kv="bf16", idx="bf16"):
    s = dict(kind="decode", B=B, seq_lens=list(lens), Hq=Hq, Hkv=Hkv, Hidx=Hidx, D=128, Di=Di,
             topk=topk, init=1, local=2, q=q, kv=kv, idx=idx, idx_value=True)
    if kv == "fp8":
        s.update(k_scale=1.0 / 16, v_scale=1.0 / 16)
    return s


def _pre(n_new, prefix, Hq=8, Hkv=2, Hidx=2, Di=128, topk=8, q="bf16", kv="bf16"):
    return dict(kind="prefill", B=len(n_new), n_new=list(n_new), prefix=list(prefix), Hq=Hq,
                Hkv=Hkv, Hidx=Hidx, D=128, Di=Di, topk=topk, init=1, local=2, q=q, kv=kv,
                idx="bf16", idx_value=True)


def _check_idx(gpu, ref, f32):
    """f32: float32 index keys and values, summed in float32 (decode); bf16
    index pools take the bf16 bounds whatever the output type, since the
    products and the probabilities enter the matrix cores in bf16."""
    parity.check_output(parity.to_np(gpu).reshape(ref.shape), ref, f32)


DECODE = {
    "ragged_di128": _dec(5, [1, 127, 129, 1000, 9000]),
    "with_empty": _dec(3, [0, 300, 5000], Hq=16, Hkv=4, Hidx=2),
    "di64_shared_idx": _dec(3, [2048, 4000, 7777], Hq=8, Hkv=2, Hidx=1, Di=64, topk=4),
    "fp8_kv": _dec(2, [30000, 12345], kv="fp8", topk=16),
    "f32": _dec(3, [1500, 4000, 9000], Hq=8, Hkv=2, Hidx=2, q="f32", kv="f32", idx="f32"),
    "long_row": _dec(2, [150001, 3000], Hq=8, Hkv=1, Hidx=1, topk=16),
}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_index_value(msa, name):
    spec = DECODE[name]
    seed = 1100 + sorted(DECODE).index(name)
    print(f"[iv_decode] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
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
    ref, _ = oracle.index_value_attention(host_view(case))
    _check_idx(idx_out, ref, spec["idx"] == "f32")


PREFILL = {
    "key_major": _pre([300, 200], [1000, 0]),
    "empty_chunk_ragged": _pre([0, 257, 129], [500, 0, 3000], Hq=16, Hkv=2, Hidx=1),
    "di64": _pre([300, 129], [2000, 700], Hq=16, Hkv=1, Hidx=1, Di=64, topk=4),
    "short_chunks": _pre([4, 1, 3, 8], [30000, 999, 5000, 127], Hq=16, Hkv=2, Hidx=2),
    "f32_q": _pre([150, 200], [1000, 2500], q="f32", kv="f32"),
    "long_prefix": _pre([40], [160000], Hq=8, Hkv=1, Hidx=1),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_index_value(msa, name):
    spec = PREFILL[name]
    seed = 1200 + sorted(PREFILL).index(name)
    print(f"[iv_prefill] {name} seed={seed}", flush=True)
    case = generate(spec, seed, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    off = msa.MsaConfig.from_spec(dict(spec, idx_value=False))
    out, lse, sel, cnt, idx_out = msa.sparse_prefill(
        cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, case.cu_seqlens_q, return_selection=True, idx_v_pool=case.idx_v_pool)
    out0, lse0, sel0, cnt0 = msa.sparse_prefill(
        off, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool, case.block_table,
        case.seq_lens, case.cu_seqlens_q, return_selection=True)
    torch.cuda.synchronize()
    for a, b in ((out, out0), (lse, lse0), (sel, sel0), (cnt, cnt0)):
        assert torch.equal(a, b)
    ref, _ = oracle.index_value_attention(host_view(case))
    _check_idx(idx_out, ref, spec["idx"] == "f32")


def test_decode_index_value_full_size(msa):
    """The batch 32 x 32768 decode workload with the index-value branch on,
    every sequence against the oracle."""
    name = "decode_b32_l32k"
    spec = dict(workload(name), idx_value=True)
    case = generate(spec, WORKLOAD_SEEDS[name], device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    print(f"[iv_decode_full] {name}", flush=True)
    out, idx_out = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                     case.idx_k_pool, case.block_table, case.seq_lens,
                                     idx_v_pool=case.idx_v_pool)
    torch.cuda.synchronize()
    ref, _ = oracle.index_value_attention(host_view(case))
    _check_idx(idx_out, ref, False)


def test_prefill_index_value_full_size_sampled(msa):
    """The 4 x 4096-token prefill over a 16384-token prefix with the branch on;
    the oracle checks the first, last and block-boundary tokens and a random
    sample of each sequence."""
    name = "prefill_4x4096_p16k"
    spec = dict(workload(name), idx_value=True)
    case = generate(spec, WORKLOAD_SEEDS[name], device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    print(f"[iv_prefill_full] {name}", flush=True)
    out, idx_out = msa.sparse_prefill(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                      case.idx_k_pool, case.block_table, case.seq_lens,
                                      case.cu_seqlens_q, idx_v_pool=case.idx_v_pool)
    torch.cuda.synchronize()
    cu = case.cu_seqlens_q.cpu().numpy()
    L = case.seq_lens.cpu().numpy()
    rng = np.random.default_rng(11)
    rows, positions = [], []
    for b in range(case.B):
        n = int(cu[b + 1] - cu[b])
        pick = sorted(set([0, n - 1, 127, 128, 2047, 2048] + rng.choice(n, 10, replace=False).tolist()))
        for i in pick:
            rows.append(int(cu[b]) + i)
            positions.append((b, int(L[b]) - n + i))
    inp = host_view(case)
    inp["idx_q"] = inp["idx_q"][rows]
    inp["positions"] = positions
    ref, _ = oracle.index_value_attention(inp)
    _check_idx(idx_out[rows], ref, False)


@pytest.mark.parametrize("idx", ["bf16", "f32"])
def test_append_index_values(msa, idx):
    """msa_append_kv with the branch on writes the index values beside the
    index keys, byte for byte as the oracle's append, and nothing else."""
    spec = dict(kind="decode", B=2, seq_lens=[300, 500], Hq=8, Hkv=2, Hidx=2, D=128,
                Di=128, topk=4, init=1, local=2, q="f32" if idx == "f32" else "bf16",
                kv="f32" if idx == "f32" else "bf16", idx=idx, idx_value=True)
    case = generate(spec, 1300, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    T = 37
    g = torch.Generator(device="cpu").manual_seed(5)
    dt = torch.float32 if idx == "f32" else torch.bfloat16
    kdt = torch.float32 if idx == "f32" else torch.bfloat16
    k_new = torch.randn((T, 2, 128), generator=g).to(kdt).cuda()
    v_new = torch.randn((T, 2, 128), generator=g).to(kdt).cuda()
    ik_new = torch.randn((T, 2, 128), generator=g).to(dt).cuda()
    iv_new = torch.randn((T, 2, 128), generator=g).to(dt).cuda()
    slots = torch.randperm(case.num_pages * 128, generator=g)[:T].to(torch.int64)
    slots[3] = -1
    before = host_view(case)
    msa.append_kv(cfg, k_new, v_new, ik_new, slots.cuda(), case.k_pool, case.v_pool,
                  case.idx_k_pool, idx_v_new=iv_new, idx_v_pool=case.idx_v_pool)
    torch.cuda.synchronize()
    after = host_view(case)
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.cpu().numpy()
    want = oracle.append_kv(before["k_pool"], before["v_pool"], before["idx_k_pool"],
                            bits(k_new), bits(v_new), bits(ik_new), slots.numpy(),
                            kv_src=spec["kv"], kv_dtype=spec["kv"], idx_dtype=idx,
                            idx_v_pool=before["idx_v_pool"], idx_v_new=bits(iv_new))
    for name, w in zip(("k_pool", "v_pool", "idx_k_pool", "idx_v_pool"), want):
        assert np.array_equal(after[name].view(np.uint8), w.view(np.uint8)), name
