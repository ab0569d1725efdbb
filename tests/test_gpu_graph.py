"""The library only enqueues kernels on the caller's stream, so its calls can be
captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.  Each replay is
checked bit for bit against an eager call on the same inputs, with eager work
and synchronisations between replays, also after the inputs change in place."""

import pytest
import torch

from synth import WORKLOAD_SEEDS, generate, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_score_amd as m
    m.load()
    return m


def _replays(run, outputs, mutate, n=4):
    """run(): enqueue the call writing `outputs`; mutate(i): change inputs in place."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(n):
        if i >= 2:
            mutate(i)
        # eager reference on the current inputs
        run()
        torch.cuda.synchronize()
        want = [o.clone() for o in outputs]
        for o in outputs:
            o.fill_(0) if o.dtype != torch.float32 else o.fill_(float("nan"))
        x = torch.randn(1 << 20, device="cuda")  # unrelated eager work
        (x * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {i}"


def test_graph_decode(msa):
    print("[graph] decode", flush=True)
    spec = dict(workload("decode_b32_l32k"), B=8)
    case = generate(spec, 61, device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    B = case.B
    out = torch.empty_like(case.q)
    lse = torch.empty((B, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, cfg.num_idx_heads, cfg.kmax), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, cfg.num_idx_heads), dtype=torch.int32, device="cuda")
    ws = msa.alloc_workspace(msa.decode_workspace_size(cfg, B, case.max_blocks), "cuda")

    def run():
        msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool,
                          case.block_table, case.seq_lens, out=out, lse=lse, sel_blocks=sel,
                          sel_count=cnt, workspace=ws, return_selection=True)

    def mutate(i):
        case.q.copy_(torch.randn_like(case.q, dtype=torch.float32).to(case.q.dtype))
        case.idx_q.copy_(torch.randn_like(case.idx_q, dtype=torch.float32).to(case.idx_q.dtype))
        case.seq_lens.sub_(i)  # shorter sequences, same table

    _replays(run, [out, lse, sel, cnt], mutate)


@pytest.mark.parametrize("name", ["prefill_4x4096_p16k", "verify_b32_q4_l32k"])
def test_graph_prefill(msa, name):
    print(f"[graph] {name}", flush=True)
    spec = workload(name)
    if name.startswith("prefill"):
        spec = dict(spec, B=2, n_new=512, prefix=3000)
    case = generate(spec, WORKLOAD_SEEDS[name], device="cuda")
    cfg = msa.MsaConfig.from_spec(spec)
    B, T = case.B, case.T
    out = torch.empty_like(case.q)
    lse = torch.empty((T, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    sel = torch.empty((T, cfg.num_idx_heads, cfg.kmax), dtype=torch.int32, device="cuda")
    cnt = torch.empty((T, cfg.num_idx_heads), dtype=torch.int32, device="cuda")
    ws = msa.alloc_workspace(msa.prefill_workspace_size(cfg, B, T, case.max_blocks), "cuda")

    def run():
        msa.sparse_prefill(cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool,
                           case.block_table, case.seq_lens, case.cu_seqlens_q, out=out, lse=lse,
                           sel_blocks=sel, sel_count=cnt, workspace=ws, return_selection=True)

    def mutate(i):
        case.q.copy_(torch.randn_like(case.q, dtype=torch.float32).to(case.q.dtype))
        case.idx_q.copy_(torch.randn_like(case.idx_q, dtype=torch.float32).to(case.idx_q.dtype))

    _replays(run, [out, lse, sel, cnt], mutate)


def test_graph_append(msa):
    print("[graph] append", flush=True)
    g = torch.Generator(device="cpu").manual_seed(3)
    cfg = msa.MsaConfig(num_q_heads=16, num_kv_heads=2, num_idx_heads=2, kv_dtype="fp8",
                        k_scale=1 / 16, v_scale=1 / 16)
    P, T = 64, 500
    pools = [torch.zeros((P, 2, 128, 128), dtype=torch.uint8, device="cuda"),
             torch.zeros((P, 2, 128, 128), dtype=torch.uint8, device="cuda"),
             torch.zeros((P, 2, 128, 128), dtype=torch.bfloat16, device="cuda")]
    new = [torch.randn((T, 2, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    slots = torch.randperm(P * 128, generator=g)[:T].cuda()

    def run():
        msa.append_kv(cfg, new[0], new[1], new[2], slots, *pools)

    def mutate(i):
        for t in new:
            t.copy_(torch.randn(t.shape, device="cuda").to(t.dtype))

    _replays(run, pools, mutate)
