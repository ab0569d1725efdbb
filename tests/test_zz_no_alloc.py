"""msa_sparse_decode_noalloc (the decode entry point that allocates nothing
and runs in the library's per-GPU scratch) against msa_sparse_decode with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller batch, each bit-identical to the workspace version (same kernels, same
launch shapes)."""

import numpy as np
import pytest
import torch

from synth import generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_score_amd as m
    m.load()
    return m


def _spec(B, lens, Hq=16, Hkv=2, Hidx=2, topk=16, kv="bf16"):
    s = dict(kind="decode", B=B, seq_lens=list(lens), Hq=Hq, Hkv=Hkv, Hidx=Hidx, D=128,
             Di=128, topk=topk, init=1, local=2, q="bf16", kv=kv, idx="bf16")
    if kv == "fp8":
        s.update(k_scale=1.0 / 16, v_scale=1.0 / 16)
    return s


def _both(msa, spec, seed):
    case = generate(spec, seed, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    B, H = case.B, cfg.num_q_heads
    ref = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool,
                            case.block_table, case.seq_lens, return_selection=True)
    out = torch.full_like(case.q, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((B, cfg.num_idx_heads, cfg.kmax), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, cfg.num_idx_heads), -7, dtype=torch.int32, device="cuda")
    msa.sparse_decode_noalloc(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                              case.idx_k_pool, case.block_table, case.seq_lens, out, lse, sel,
                              cnt)
    torch.cuda.synchronize()
    return ref, (out, lse, sel, cnt)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_decode_equals_workspace_decode(msa, kv):
    big = _spec(8, [300, 4000, 20000, 129, 65536, 1, 9000, 33000], kv=kv)
    small = _spec(3, [5000, 128, 700], Hq=8, Hkv=2, Hidx=1, topk=4, kv=kv)
    for spec, seed in ((big, 71), (small, 72)):
        print(f"noalloc decode: kv={kv} B={spec['B']} lens={spec['seq_lens']}", flush=True)
        ref, got = _both(msa, spec, seed)
        for r, g, name in zip(ref, got, ("out", "lse", "sel", "cnt")):
            assert torch.equal(r, g), name
        assert np.isfinite(got[0].float().cpu().numpy()).all()


def test_noalloc_decode_refuses_a_batch_past_its_scratch(msa):
    spec = _spec(2, [1000, 2000])
    case = generate(spec, 73, device="cuda", max_blocks=8192)
    cfg = msa.MsaConfig.from_spec(spec)
    # 2 sequences x 8192 blocks fit; 2048 sequences of 8192 blocks would not
    big_table = case.block_table.repeat(1024, 1)
    big_lens = case.seq_lens.repeat(1024)
    out = torch.empty((2048, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msa.MsaError) as e:
        msa.sparse_decode_noalloc(cfg, out, case.idx_q.repeat(1024, 1, 1), case.k_pool,
                                  case.v_pool, case.idx_k_pool, big_table, big_lens, out)
    assert "scratch" in str(e.value)
