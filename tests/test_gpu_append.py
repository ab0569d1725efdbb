"""GPU parity of the paged append (msa_append_kv) against the oracle, through
the C ABI: every byte of every pool, and the append -> decode flow."""

import numpy as np
import pytest
import torch

import oracle
import parity
from synth import generate, host_view

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_score_amd as m
    m.load()
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


CASES = {
    # name: (kv pool dtype, idx dtype, Hkv, Hidx, Di, k_scale, v_scale)
    "bf16": ("bf16", "bf16", 2, 2, 128, 1.0, 1.0),
    "bf16_idx_f32_di64": ("bf16", "f32", 4, 2, 64, 1.0, 1.0),
    "f32": ("f32", "f32", 2, 1, 128, 1.0, 1.0),
    "fp8": ("fp8", "bf16", 2, 2, 128, 1 / 16, 1 / 16),
    "fp8_odd_scales": ("fp8", "bf16", 1, 1, 64, 0.37, 0.11),
    "fp8_e5m2": ("fp8_e5m2", "bf16", 2, 2, 128, 1 / 16, 1 / 16),
    "fp8_e5m2_odd_scales": ("fp8_e5m2", "bf16", 1, 1, 64, 0.37, 0.011),
}


@pytest.mark.parametrize("name", list(CASES))
def test_append_matches_oracle_bytes(msa, name):
    kv, idx, Hkv, Hidx, Di, ks, vs = CASES[name]
    print(f"[append] {name}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(5)
    P, D, T = 40, 128, 300
    src_dt = torch.float32 if kv == "f32" else torch.bfloat16
    idx_dt = torch.float32 if idx == "f32" else torch.bfloat16

    def new_rows(shape, dt):
        # N(0,1), with some rows far outside e4m3's range and some tiny
        x = torch.randn(shape, generator=g)
        x[::7] *= 300.0
        x[5::13] *= 3e4          # past e5m2's largest finite value once scaled
        x[3::11] *= 1e-4
        return x.to(dt)

    def pool(shape, dt):
        if dt.startswith("fp8"):
            return torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
        return torch.randn(shape, generator=g).to(src_dt if dt != "idx" else idx_dt)

    k_pool = pool((P, Hkv, 128, D), kv)
    v_pool = pool((P, Hkv, 128, D), kv)
    ik_pool = pool((P, Hidx, 128, Di), "idx")
    k_new, v_new = new_rows((T, Hkv, D), src_dt), new_rows((T, Hkv, D), src_dt)
    # exact ties of e4m3 rounding in the fp8 cases: midpoints of neighbouring codes times scale
    tab = oracle.fp8_e5m2_table() if kv == "fp8_e5m2" else oracle.fp8_e4m3fn_table()
    mids = torch.tensor((tab[0x10:0x20] + tab[0x11:0x21]) / 2.0, dtype=torch.float32)
    k_new[0, 0, :16] = (mids * ks).to(src_dt)
    ik_new = new_rows((T, Hidx, Di), idx_dt)
    slots = torch.randperm(P * 128, generator=g)[:T].to(torch.int64)
    slots[5] = -1
    slots[17] = P * 128          # past the pool: skipped
    slots[18] = -(1 << 40)

    dev = torch.device("cuda")
    pools = [t.to(dev) for t in (k_pool, v_pool, ik_pool)]
    cfg = msa.MsaConfig(num_q_heads=Hkv * 4, num_kv_heads=Hkv, num_idx_heads=Hidx,
                        idx_dim=Di, q_dtype="f32" if kv == "f32" else "bf16", kv_dtype=kv,
                        idx_dtype=idx, k_scale=ks, v_scale=vs)
    msa.append_kv(cfg, k_new.to(dev), v_new.to(dev), ik_new.to(dev), slots.to(dev), *pools)
    torch.cuda.synchronize()

    src = "f32" if kv == "f32" else "bf16"
    want = oracle.append_kv(_bits(k_pool), _bits(v_pool), _bits(ik_pool), _bits(k_new),
                            _bits(v_new), _bits(ik_new), slots.numpy(), kv_src=src,
                            kv_dtype=kv, idx_dtype=idx, k_scale=ks, v_scale=vs)
    for got, ref, what in zip(pools, want, ("k_pool", "v_pool", "idx_k_pool")):
        g_np = _bits(got)
        # byte-exact: compare raw bit patterns (pools hold NaN bit patterns too)
        bad = g_np.view(np.uint8) != np.ascontiguousarray(ref).view(np.uint8)
        assert not bad.any(), f"{what}: {int(bad.sum())} bytes differ"


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_then_decode(msa, kv):
    """The serving order: the current token's K, V and index key are appended
    into their slots (through the shuffled block table), then decoded; the
    output equals the oracle's on the fully written cache."""
    spec = dict(kind="decode", B=3, seq_lens=[5000, 129, 33000], Hq=16, Hkv=2, Hidx=2, D=128,
                Di=128, topk=8, init=1, local=2, q="bf16", kv=kv, idx="bf16")
    if kv == "fp8":
        spec.update(k_scale=1 / 16, v_scale=1 / 16)
    print(f"[append_decode] {kv}", flush=True)
    case = generate(spec, 77, device="cuda")
    ref_inp = host_view(case)
    cfg = msa.MsaConfig.from_spec(spec)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    bt = case.block_table.cpu().numpy()
    pages = np.array([bt[b, (L - 1) // 128] for b, L in enumerate(lens)], dtype=np.int64)
    slots = torch.tensor(pages * 128 + (lens - 1) % 128, dtype=torch.int64, device="cuda")
    # the new tokens' rows, as the model would produce them (bf16; for an fp8
    # pool, values whose quotient by the scale is the stored code)
    def rows(pool, scale):
        r = pool[slots // 128, :, slots % 128, :]
        if kv == "fp8" and pool is not case.idx_k_pool:
            return (r.view(torch.float8_e4m3fn).float() * scale).to(torch.bfloat16)
        return r.clone()
    k_new, v_new = rows(case.k_pool, case.k_scale), rows(case.v_pool, case.v_scale)
    ik_new = rows(case.idx_k_pool, 1.0)
    # wipe the slots (NaN / poison), then append
    for pool in (case.k_pool, case.v_pool):
        pool[slots // 128, :, slots % 128, :] = (0x7F if kv == "fp8" else float("nan"))
    case.idx_k_pool[slots // 128, :, slots % 128, :] = 1e4
    msa.append_kv(cfg, k_new, v_new, ik_new, slots, case.k_pool, case.v_pool, case.idx_k_pool)
    out, lse, sel, cnt = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                           case.idx_k_pool, case.block_table, case.seq_lens,
                                           return_selection=True)
    torch.cuda.synchronize()
    inp = host_view(case)
    for key in ("k_pool", "v_pool", "idx_k_pool"):
        assert np.array_equal(inp[key].view(np.uint8), ref_inp[key].view(np.uint8)), key
    ora = oracle.sparse_attention(ref_inp)
    gsel, gcnt = parity.to_np(sel), parity.to_np(cnt)
    pos = oracle.query_positions(ref_inp["seq_lens"], None)
    parity.check_selection(gsel, gcnt, ora["scores"], ora["sel"], ora["count"], pos,
                           spec["init"], spec["local"])
    ora_out, _ = oracle.attend(ref_inp, gsel, gcnt)
    parity.check_output(parity.to_np(out), ora_out, False)


def test_append_more_tokens_than_one_grid_row(msa):
    """70000 tokens in one call (tokens lie on the grid's x dimension)."""
    print("[append_many] 70000 tokens", flush=True)
    g = torch.Generator(device="cpu").manual_seed(12)
    P, T, Hkv, Hidx, Di = 600, 70000, 2, 1, 64
    pools = [torch.randn((P, Hkv, 128, 128), generator=g).to(torch.bfloat16),
             torch.randn((P, Hkv, 128, 128), generator=g).to(torch.bfloat16),
             torch.randn((P, Hidx, 128, Di), generator=g).to(torch.bfloat16)]
    new = [torch.randn((T, Hkv, 128), generator=g).to(torch.bfloat16),
           torch.randn((T, Hkv, 128), generator=g).to(torch.bfloat16),
           torch.randn((T, Hidx, Di), generator=g).to(torch.bfloat16)]
    slots = torch.randperm(P * 128, generator=g)[:T].to(torch.int64)
    cfg = msa.MsaConfig(num_q_heads=8, num_kv_heads=Hkv, num_idx_heads=Hidx, idx_dim=Di)
    dev_pools = [t.cuda() for t in pools]
    msa.append_kv(cfg, *[t.cuda() for t in new], slots.cuda(), *dev_pools)
    torch.cuda.synchronize()
    want = oracle.append_kv(*[_bits(t) for t in pools], *[_bits(t) for t in new], slots.numpy(),
                            kv_src="bf16", kv_dtype="bf16", idx_dtype="bf16")
    for got, ref in zip(dev_pools, want):
        assert np.array_equal(_bits(got), ref)
