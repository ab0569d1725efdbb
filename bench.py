"""Benchmark of block-sparse attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-configs]
                    [--no-cpu-baseline]

Default: decode of 64 sequences with lengths drawn uniformly from 4096 to
131072 tokens (the largest decode workload on one GPU) is the headline line;
the four other workloads of the method's configurations are measured after it
in the same run and reported under "configs": decode 2 x 2048, decode
32 x 32768, fp8-e4m3 decode 32 x 65536 and chunked prefill 4 x 4096 over a
16384-token prefix.  ``--workload NAME`` makes NAME the headline (prefill and
append workloads report tokens/s); ``--no-configs`` measures the headline
alone (profiling runs).  In the default run every workload is measured in a
process of its own (this process only starts them and joins their lines), so
that no workload runs in memory the previous one allocated and freed; with
``--no-configs`` the measurement runs in this process.

A decode step is one msa_sparse_decode call (score every block of the index keys,
select, split-K attend over the selected blocks, combine) over one batch of
synthetic inputs already resident in HBM; a prefill step is one
msa_sparse_prefill call.  Before every timed step a 1 GiB buffer is
overwritten so that no input is served from the L2 or the 256 MB Infinity
Cache; HIP events on the library's stream bracket each step.

Prints ONE JSON line: queries/s (value), achieved HBM GB/s on the touched
bytes of the step, the roofline of the dominant kernel (the index-key scan,
timed standalone through msa_block_score on the same inputs) and the fp64
oracle timed on the host cores over a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "sparse-decode queries/sec + achieved HBM GB/s (touched bytes) at 1 MI355X"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "decode_b64_lvar"
# the other workloads of the method's configurations, reported beside the headline
SUB_CONFIGS = ["decode_b2_l2048", "decode_b32_l32k", "decode_fp8_b32_l64k",
               "prefill_4x4096_p16k"]
MFMA_BF16_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sub-config", action="store_true",
                    help="measure as a workload beside the headline (no warm steps)")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a read+write kernel over 1 GiB (HBM counter calibration)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("SCAN_RD", "SCAN_WR", "COPY_RD",
                                                          "COPY_WR"),
                    help="rocprofv3 --pmc output folders -> profiles/ HBM traffic summary "
                         "of the --workload decode scan")
    return ap.parse_args()


def elem_bytes(dt: str) -> float:
    # MX-fp4 / MX-fp6: half a byte / three quarters of a byte per element,
    # plus one scale byte per 32
    return {"bf16": 2, "f32": 4, "fp8": 1, "fp8_e5m2": 1, "mxfp4": 17 / 32, "mxfp6": 25 / 32}[dt]


def step_bytes(spec, seq_lens, sel, cnt):
    """Algorithmic bytes of one decode step (what the method must move)."""
    B, Hq, Hkv, Hidx = spec["B"], spec["Hq"], spec["Hkv"], spec["Hidx"]
    D, Di = spec["D"], spec["Di"]
    ei, ekv, eq = elem_bytes(spec["idx"]), elem_bytes(spec["kv"]), elem_bytes(spec["q"])
    L = seq_lens.astype(np.int64)
    nb = (L + 127) // 128
    idx_keys = int((Hidx * L * Di * ei).sum())
    gpi = Hkv // Hidx
    kv = 0
    for b in range(B):
        for g in range(Hkv):
            h = g // gpi
            for j in sel[b, h, : cnt[b, h]]:
                valid = min(128, int(L[b]) - 128 * int(j))
                kv += valid * D * 2 * ekv
    small = int(B * Hq * D * 2 * eq + B * Hidx * Di * eq + 4 * (nb.sum() + Hkv * cnt.sum()))
    if spec.get("idx_value"):
        # the index values of every visible token, and the index output
        idx_keys *= 2
        small += B * Hidx * Di * eq
    return idx_keys, int(kv), small


def score_kernel_bytes(spec, seq_lens, max_blocks):
    """Algorithmic bytes of one standalone scoring launch: index keys of every
    visible token, the index queries, the block table rows read and the score
    rows written."""
    B, Hidx, Di = spec["B"], spec["Hidx"], spec["Di"]
    ei = elem_bytes(spec["idx"])
    L = seq_lens.astype(np.int64)
    nb = (L + 127) // 128
    return int((Hidx * L * Di * ei).sum() + B * Hidx * Di * ei + 4 * nb.sum() * Hidx
               + 4 * B * Hidx * max_blocks)


def prefill_flops(spec, seq_lens, cu, sel_valid):
    """Algorithmic flops of one prefill step: the causal index-score GEMM
    (2 * Di per visible token per query and index head) and the attention over
    each query's selected visible tokens (4 * D per token and q head: q.k and
    p.v).  ``sel_valid`` sums the selected visible tokens over (query, index
    head); every index head serves Hq / Hidx q heads."""
    Hq, Hidx, D, Di = spec["Hq"], spec["Hidx"], spec["D"], spec["Di"]
    score = 0
    for b in range(len(seq_lens)):
        n = int(cu[b + 1] - cu[b])
        p0 = int(seq_lens[b]) - n
        score += n * (p0 + 1) + n * (n - 1) // 2   # sum of (p + 1) over the queries
    score *= 2 * Hidx * Di
    attn = 4 * D * (Hq // Hidx) * int(sel_valid)
    return score, attn


def selected_valid_tokens(seq_lens, cu, sel, cnt):
    """Sum over (query, index head) of the visible tokens of the selected blocks."""
    tot = 0
    for b in range(len(seq_lens)):
        n = int(cu[b + 1] - cu[b])
        L = int(seq_lens[b])
        for i in range(n):
            t = int(cu[b]) + i
            p = L - n + i
            for h in range(sel.shape[1]):
                js = sel[t, h, : cnt[t, h]].astype(np.int64)
                tot += int(np.minimum(128, p + 1 - 128 * js).sum())
    return tot


def cpu_baseline(case, spec, seconds):
    """The oracle as it stands, on the same inputs, sequence by sequence."""
    import torch  # noqa: F401

    import oracle
    from synth import host_view

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    B = case.B
    lens = case.seq_lens.cpu().numpy()
    bt = case.block_table.cpu().numpy()
    # Sequences in order, wrapping round the batch until the time target is met.
    done, t_used, n = 0, 0.0, 1
    while t_used < seconds and done < 64 * B:
        start = done % B
        rows = list(range(start, min(B, start + n)))
        pages = np.unique(bt[rows].reshape(-1))
        pages = pages[pages >= 0]
        inp = host_view(case, pages=pages)
        sub = dict(inp)
        sub["q"] = inp["q"][rows]
        sub["idx_q"] = inp["idx_q"][rows]
        sub["block_table"] = inp["block_table"][rows]
        sub["seq_lens"] = inp["seq_lens"][rows]
        t0 = time.perf_counter()
        oracle.sparse_attention(sub)
        t_used += time.perf_counter() - t0
        done += len(rows)
        n = min(2 * n, 8)
    return dict(value=done / t_used, unit="queries/s", cores=int(blas_threads),
                host_cpus=len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"{done} sequences ({done / B:.1f} passes over the {B} of "
                       f"{spec['name']}, all heads), {t_used:.1f} s of fp64 numpy")


# ---------------------------------------------------------------- HBM traffic
#
# The scan's HBM bytes come from the L2-to-memory request counters of two
# rocprofv3 --pmc passes (reads, then writes), scaled by what the same
# counters read for a kernel of known traffic (the copy probe: 1 GiB read and
# 1 GiB written).  gfx950 issues 32-, 64- and 128-byte read requests; the
# stock FETCH_SIZE expression counts the 128-byte ones only through
# TCC_BUBBLE, which the scan's non-temporal loads do not raise, so reads are
# counted here from TCC_EA0_RDREQ_128B / _32B directly.
TRAFFIC_RD = ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_EA0_RDREQ_32B_sum",
              "TCC_BUBBLE_sum"]
TRAFFIC_WR = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"]
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


COPY_PROBE_BYTES = 1 << 30
# The kernels whose counters make a workload's roofline traffic, and the
# sources a measurement stays valid for: the decode index scan; the prefill
# attention stage (k2q lists, key-major tiles, forced blocks, combine), per
# step.
SCAN_SOURCES = ["msa_score.h", "msa_score.hip", "msa_device.h", "msa_internal.h"]
STAGE_SOURCES = ["msa_prefill_attend.hip", "msa_device.h", "msa_internal.h"]
STAGE_KERNELS = ["k2q_count_kernel", "k2q_scan_kernel", "k2q_fill_kernel",
                 "prefill_attend_kernel", "prefill_forced_kernel", "prefill_combine_kernel"]


def traffic_json(workload_name: str) -> str:
    from synth import workload
    part = "scan" if workload(workload_name)["kind"] == "decode" else "attention"
    return os.path.join(PROFILES, f"{workload_name}_{part}_hbm_traffic.json")


def source_hash(names=SCAN_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "block_sparse_attention_score_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def scan_source_hash() -> str:
    return source_hash(SCAN_SOURCES)


def copy_probe():
    """1 GiB read and 1 GiB written by one elementwise kernel, three times."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES}), flush=True)


def _counters(folder, kernel_substr):
    """Per-dispatch counter values of the kernels whose name contains kernel_substr."""
    import csv
    import glob
    per = {}
    paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    # one profiled run: the newest file (a folder reused across runs keeps older ones)
    for path in sorted(paths, key=os.path.getmtime)[-1:]:
        for r in csv.DictReader(open(path)):
            if kernel_substr not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel matching {kernel_substr!r} under {folder}")
    return list(per.values())


def _read_bytes(c):
    rd, r128, r32 = c["TCC_EA0_RDREQ_sum"], c["TCC_EA0_RDREQ_128B_sum"], c["TCC_EA0_RDREQ_32B_sum"]
    return 128 * r128 + 64 * (rd - r128 - r32) + 32 * r32


def _fetch_size_bytes(c):  # the stock FETCH_SIZE expression, for comparison
    rd, bub, r32 = c["TCC_EA0_RDREQ_sum"], c["TCC_BUBBLE_sum"], c["TCC_EA0_RDREQ_32B_sum"]
    return 128 * bub + 64 * (rd - bub - r32) + 32 * r32


def _write_bytes(c):
    wr, w64 = c["TCC_EA0_WRREQ_sum"], c["TCC_EA0_WRREQ_64B_sum"]
    return 64 * w64 + 32 * (wr - w64)


def traffic_summary(name, scan_rd, scan_wr, copy_rd, copy_wr):
    """Write the calibrated HBM traffic of workload ``name`` to profiles/
    (JSON for bench.py, Markdown for readers): the index scan of a decode
    workload, the attention stage of a prefill workload."""
    from synth import WORKLOAD_SEEDS, workload
    from synth.inputs import _draw_seq_lens

    if workload(name)["kind"] == "prefill":
        return stage_traffic_summary(name, scan_rd, scan_wr, copy_rd, copy_wr)

    med = lambda xs: float(np.median(xs))
    s_rd = _counters(scan_rd, "decode_score_kernel")
    s_wr = _counters(scan_wr, "decode_score_kernel")
    c_rd = _counters(copy_rd, "neg")
    c_wr = _counters(copy_wr, "neg")
    f_rd = COPY_PROBE_BYTES / med([_read_bytes(c) for c in c_rd])
    f_wr = COPY_PROBE_BYTES / med([_write_bytes(c) for c in c_wr])
    rd = med([_read_bytes(c) for c in s_rd]) * f_rd
    wr = med([_write_bytes(c) for c in s_wr]) * f_wr
    stock = med([_fetch_size_bytes(c) for c in s_rd])
    spec = workload(name)
    lens = _draw_seq_lens(spec, WORKLOAD_SEEDS[name]).numpy().astype(np.int64)
    alg = score_kernel_bytes(spec, lens, int(((lens + 127) // 128).max()))
    res = {"kernel": "decode_score_kernel", "workload": name,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "traffic_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": alg,
           "copy_factor_read": f_rd, "copy_factor_write": f_wr, "stock_fetch_size_bytes": stock,
           "dispatches": [len(s_rd), len(s_wr)], "source_sha256": scan_source_hash()}
    path = traffic_json(name)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    lens_txt = (f"L = {lens[0]}" if (lens == lens[0]).all()
                else f"L from {lens.min()} to {lens.max()}, mean {lens.mean():.0f}")
    with open(path[:-5] + ".md", "w") as f:
        f.write(
            f"# HBM traffic of the decode index scan, {name} (B={spec['B']}, {lens_txt}, "
            f"{spec['Hidx']} index heads, Di={spec['Di']})\n\n"
            "Commands (run from the repository root on one MI355X; each pass alone):\n\n"
            "    cd /tmp && export TMPDIR=/tmp\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_RD)} --output-format csv -d <scan_rd> -- python3 <repo>/bench.py --workload {name} --no-configs --steps 3 --warmup 1 --no-cpu-baseline\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_WR)} --output-format csv -d <scan_wr> -- python3 <repo>/bench.py --workload {name} --no-configs --steps 3 --warmup 1 --no-cpu-baseline\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_RD)} --output-format csv -d <copy_rd> -- python3 <repo>/bench.py --copy-probe\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_WR)} --output-format csv -d <copy_wr> -- python3 <repo>/bench.py --copy-probe\n"
            f"    python3 bench.py --workload {name} --traffic-summary <scan_rd> <scan_wr> <copy_rd> <copy_wr>\n\n"
            "Bytes per launch are 128 x RDREQ_128B + 64 x (RDREQ - RDREQ_128B - RDREQ_32B) + 32 x RDREQ_32B\n"
            "(reads) and 64 x WRREQ_64B + 32 x (WRREQ - WRREQ_64B) (writes), medians over the dispatches,\n"
            "scaled by the copy probe (1 GiB read and written by one elementwise kernel).\n\n"
            "| quantity | value |\n|---|---|\n"
            f"| scan reads per launch | {rd / 1e6:.1f} MB |\n"
            f"| scan writes per launch | {wr / 1e6:.3f} MB |\n"
            f"| algorithmic bytes per launch | {alg / 1e6:.1f} MB |\n"
            f"| copy-probe factor, reads / writes | {f_rd:.3f} / {f_wr:.3f} |\n"
            f"| stock FETCH_SIZE expression for the scan | {stock / 1e6:.1f} MB |\n"
            f"| dispatches (read pass, write pass) | {len(s_rd)}, {len(s_wr)} |\n"
            f"| sha256 of {', '.join(SCAN_SOURCES)} | `{res['source_sha256'][:16]}...` |\n")
    print(json.dumps(res))


def stage_traffic_summary(name, pf_rd, pf_wr, copy_rd, copy_wr):
    """Prefill: calibrated HBM bytes per step of each attention-stage kernel
    and their sum (the stage's roofline traffic), with the scoring and
    selection kernels beside them for reference."""
    med = lambda xs: float(np.median(xs))
    c_rd = _counters(copy_rd, "neg")
    c_wr = _counters(copy_wr, "neg")
    f_rd = COPY_PROBE_BYTES / med([_read_bytes(c) for c in c_rd])
    f_wr = COPY_PROBE_BYTES / med([_write_bytes(c) for c in c_wr])
    rows = {}
    for k in STAGE_KERNELS + ["prefill_score_kernel", "select_wave_kernel"]:
        rd = med([_read_bytes(c) for c in _counters(pf_rd, k)]) * f_rd
        wr = med([_write_bytes(c) for c in _counters(pf_wr, k)]) * f_wr
        rows[k] = {"read": rd, "write": wr}
    total = sum(rows[k]["read"] + rows[k]["write"] for k in STAGE_KERNELS)
    res = {"kernel": "prefill attention stage", "workload": name, "kernels": rows,
           "traffic_bytes_per_launch": total, "copy_factor_read": f_rd,
           "copy_factor_write": f_wr, "source_sha256": source_hash(STAGE_SOURCES)}
    path = traffic_json(name)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    table = "".join(f"| `{k}` | {v['read'] / 1e6:.1f} | {v['write'] / 1e6:.1f} |\n"
                    for k, v in rows.items())
    with open(path[:-5] + ".md", "w") as f:
        f.write(
            f"# HBM traffic of the prefill attention stage, {name}\n\n"
            "Commands (run from the repository root on one MI355X; each pass alone):\n\n"
            "    cd /tmp && export TMPDIR=/tmp\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_RD)} --output-format csv -d <pf_rd> -- python3 <repo>/bench.py --workload {name} --no-configs --steps 3 --warmup 1 --no-cpu-baseline\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_WR)} --output-format csv -d <pf_wr> -- python3 <repo>/bench.py --workload {name} --no-configs --steps 3 --warmup 1 --no-cpu-baseline\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_RD)} --output-format csv -d <copy_rd> -- python3 <repo>/bench.py --copy-probe\n"
            f"    rocprofv3 --pmc {' '.join(TRAFFIC_WR)} --output-format csv -d <copy_wr> -- python3 <repo>/bench.py --copy-probe\n"
            f"    python3 bench.py --workload {name} --traffic-summary <pf_rd> <pf_wr> <copy_rd> <copy_wr>\n\n"
            "L2-to-memory bytes per launch (medians over the dispatches, the same byte counts and\n"
            "copy-probe scaling as the decode scan's summary), in MB:\n\n"
            "| kernel | read | write |\n|---|---|---|\n" + table +
            f"\nAttention stage (the first five rows) per step: {total / 1e6:.1f} MB.  Copy-probe factors "
            f"{f_rd:.3f} (reads), {f_wr:.3f} (writes).  sha256 of {', '.join(STAGE_SOURCES)}: "
            f"`{res['source_sha256'][:16]}...`\n")
    print(json.dumps(res))


def measured_traffic(name):
    """The calibrated roofline traffic per launch of workload ``name`` (decode:
    the index scan; prefill: the attention stage per step), while the sources
    are the ones it was measured on; else None."""
    try:
        with open(traffic_json(name)) as f:
            t = json.load(f)
    except OSError:
        return None
    from synth import workload
    names = SCAN_SOURCES if workload(name)["kind"] == "decode" else STAGE_SOURCES
    if t.get("source_sha256") != source_hash(names):
        return None
    return t["traffic_bytes_per_launch"]


def device_info(dev):
    import torch
    props = torch.cuda.get_device_properties(dev)
    return {"device": torch.cuda.get_device_name(dev),
            "device_arch": getattr(props, "gcnArchName", "unknown")}


def timed_steps(fn, n, flush, stream):
    """n calls of fn, each after a 1 GiB overwrite, HIP events on ``stream``
    around each call; returns the per-call times in ms."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i in range(n):
        flush.fill_(i)
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def sub_entry(res):
    """What a workload measured beside the headline reports."""
    keep = ("value", "unit", "ms_per_step", "ms_per_step_median", "hbm_gbps", "hbm_frac",
            "touched_bytes", "stages_ms", "mfma_tflops", "mfma_frac", "flops", "roofline")
    out = {k: res[k] for k in keep if k in res}
    out["config"] = res["config"]
    return out


def main():
    args = parse()
    if args.traffic_summary:
        return traffic_summary(args.workload, *args.traffic_summary)
    if args.copy_probe:
        return copy_probe()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    from synth import workload

    if not args.no_configs and args.workload == DEFAULT_WORKLOAD:
        # (this process does not touch the GPU: the children measure)
        res = measure_in_child(args, args.workload, headline=True)
        res["configs"] = {}
        for name in SUB_CONFIGS:
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            res["configs"][name] = sub_entry(measure_in_child(args, name, headline=False))
        print(json.dumps(res), flush=True)
        return
    measure = {"decode": measure_decode, "prefill": measure_prefill, "append": measure_append}
    spec = workload(args.workload)
    res = measure[spec["kind"]](args, args.workload, headline=not args.sub_config)
    print(json.dumps(res), flush=True)


def measure_in_child(args, name, headline):
    """One workload measured by ``bench.py --workload name --no-configs`` in a
    child process; its JSON line."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--no-configs",
           "--steps", str(args.steps), "--warmup", str(args.warmup),
           "--cpu-seconds", str(args.cpu_seconds)]
    if not headline:
        cmd += ["--sub-config", "--no-cpu-baseline"]
    elif args.no_cpu_baseline:
        cmd.append("--no-cpu-baseline")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if r.returncode != 0:
        print(r.stdout, file=sys.stderr)
        raise SystemExit(f"bench.py: measuring {name} failed (exit {r.returncode})")
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def measure_decode(args, name, headline):
    """One decode workload: step time over K cold-cache steps, touched bytes,
    the standalone index scan (the dominant kernel); on the headline also the
    warm step and the oracle on the host cores."""
    import torch

    import block_sparse_attention_score_amd as msa
    from synth import WORKLOAD_SEEDS, generate, workload

    spec = workload(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = generate(spec, WORKLOAD_SEEDS[name], device=dev)
    cfg = msa.MsaConfig.from_spec(spec)
    B, MB = case.B, case.max_blocks
    ws = msa.alloc_workspace(msa.decode_workspace_size(cfg, B, MB), dev)
    out = torch.empty_like(case.q)
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def step():
        msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool,
                          case.block_table, case.seq_lens, out=out, workspace=ws,
                          idx_v_pool=case.idx_v_pool)

    # selection of this batch, for the touched-bytes count
    _, _, sel, cnt = msa.sparse_decode(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                       case.idx_k_pool, case.block_table, case.seq_lens,
                                       workspace=ws, return_selection=True,
                                       idx_v_pool=case.idx_v_pool)[:4]
    torch.cuda.synchronize()
    lens = case.seq_lens.cpu().numpy()
    idx_b, kv_b, small_b = step_bytes(spec, lens, sel.cpu().numpy(), cnt.cpu().numpy())
    total_b = idx_b + kv_b + small_b

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, cold caches, events on the library's stream
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    step_ms = timed_steps(step, args.steps, flush, stream)
    t_wall = time.perf_counter() - t_wall0
    ms = float(step_ms.mean())

    # ---- dominant kernel: the index-key scan, standalone, cold caches
    scores = torch.empty((B, cfg.num_idx_heads, MB), dtype=torch.float32, device=dev)
    k_ms = float(timed_steps(lambda: msa.block_score(cfg, case.idx_q, case.idx_k_pool,
                                                     case.block_table, case.seq_lens,
                                                     scores=scores),
                             args.steps, flush, stream).mean())
    k_bytes = score_kernel_bytes(spec, lens, MB)
    k_gbs = k_bytes / (k_ms * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": B / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["kv"] if spec["kv"] != "bf16" else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "seq_lens": spec["seq_lens"],
                   "q_heads": spec["Hq"], "kv_heads": spec["Hkv"], "idx_heads": spec["Hidx"],
                   "head_dim": spec["D"], "idx_dim": spec["Di"], "topk": spec["topk"],
                   "init": spec["init"], "local": spec["local"], "kv_dtype": spec["kv"],
                   "page": 128, "parallelism": "none"},
        "hbm_gbps": total_b / (ms * 1e-3) / 1e9,
        "hbm_frac": total_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "touched_bytes": {"idx_keys": idx_b, "selected_kv": kv_b, "small": small_b},
        "ms_per_step_median": float(np.median(step_ms)),
        "wall_s_timed_region": t_wall,
        "roofline": {"kernel": "decode_score_kernel (index-key scan)", "bound": "hbm",
                     "achieved": k_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(name),
                     "bytes_per_launch": k_bytes, "ms_per_launch": k_ms},
        **device_info(dev),
    }
    if headline:
        # warm back-to-back steps (context only)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        res["ms_per_step_warm"] = e0.elapsed_time(e1) / args.steps
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline(case, spec, args.cpu_seconds)
    return res


def measure_prefill(args, name, headline):
    """Chunked prefill: tokens/s of msa_sparse_prefill, with the index-score
    GEMM and the selection timed standalone on the same inputs (attention is
    the remainder of the step)."""
    import torch

    import block_sparse_attention_score_amd as msa
    from synth import WORKLOAD_SEEDS, generate, workload

    spec = workload(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = generate(spec, WORKLOAD_SEEDS[name], device=dev)
    cfg = msa.MsaConfig.from_spec(spec)
    B, MB, T = case.B, case.max_blocks, case.T
    ws = msa.alloc_workspace(msa.prefill_workspace_size(cfg, B, T, MB), dev)
    out = torch.empty_like(case.q)
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def step():
        msa.sparse_prefill(cfg, case.q, case.idx_q, case.k_pool, case.v_pool, case.idx_k_pool,
                           case.block_table, case.seq_lens, case.cu_seqlens_q, out=out,
                           workspace=ws, idx_v_pool=case.idx_v_pool)

    _, _, sel, cnt = msa.sparse_prefill(cfg, case.q, case.idx_q, case.k_pool, case.v_pool,
                                        case.idx_k_pool, case.block_table, case.seq_lens,
                                        case.cu_seqlens_q, workspace=ws, return_selection=True,
                                        idx_v_pool=case.idx_v_pool)[:4]
    torch.cuda.synchronize()
    lens = case.seq_lens.cpu().numpy()
    cu = case.cu_seqlens_q.cpu().numpy()
    valid = selected_valid_tokens(lens, cu, sel.cpu().numpy(), cnt.cpu().numpy())
    f_score, f_attn = prefill_flops(spec, lens, cu, valid)
    # index-value branch: q.k over the same (query, visible token) pairs as
    # the scoring, and p.v over them again
    f_iv = 2 * f_score if spec.get("idx_value") else 0

    def timed(fn, n):
        return timed_steps(fn, n, flush, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    step_ms = timed(step, args.steps)
    t_wall = time.perf_counter() - t_wall0
    ms = float(step_ms.mean())
    scores = torch.empty((T, cfg.num_idx_heads, MB), dtype=torch.float32, device=dev)
    score_ms = float(timed(lambda: msa.block_score(cfg, case.idx_q, case.idx_k_pool,
                                                   case.block_table, case.seq_lens,
                                                   cu_seqlens_q=case.cu_seqlens_q,
                                                   scores=scores), args.steps).mean())
    sel_ms = float(timed(lambda: msa.select_blocks(cfg, scores, case.seq_lens,
                                                   cu_seqlens_q=case.cu_seqlens_q),
                         args.steps).mean())
    attn_ms = max(ms - score_ms - sel_ms, 1e-6)
    # short chunks (at most 8 new tokens per sequence on average) take the
    # page-scan path: HBM-bound like decode
    short = T <= 8 * B
    peak = MFMA_BF16_PEAK_TFLOPS
    score_tf = f_score / (score_ms * 1e-3) / 1e12
    attn_tf = f_attn / (attn_ms * 1e-3) / 1e12
    dominant = "attention" if attn_ms >= score_ms else "score"
    roof = {"kernel": "prefill attention stage (k2q lists, key-major MFMA tiles, forced blocks, "
                      "combine)",
            "bound": "mfma", "achieved": attn_tf, "peak": peak, "unit": "TFLOP/s",
            "frac": attn_tf / peak, "traffic": measured_traffic(name), "flops_per_launch": f_attn,
            "ms_per_launch": attn_ms} if dominant == "attention" else \
           {"kernel": "prefill_score_kernel (causal index-score GEMM)", "bound": "mfma",
            "achieved": score_tf, "peak": peak, "unit": "TFLOP/s", "frac": score_tf / peak,
            "traffic": None, "flops_per_launch": f_score, "ms_per_launch": score_ms}
    if short:
        idx_b, kv_b, small_b = chunk_touched_bytes(spec, lens, cu, sel.cpu().numpy(),
                                                   cnt.cpu().numpy())
        scan_b = idx_b + int(T * cfg.num_idx_heads * cfg.idx_dim * 2 + 4 * (B * MB))
        roof = {"kernel": "multi_score_kernel (index-key scan, four queries per pass)",
                "bound": "hbm", "achieved": scan_b / (score_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": scan_b / (score_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                "bytes_per_launch": scan_b, "ms_per_launch": score_ms}
    res = {
        "metric": ("multi-token decode tokens/sec + achieved HBM GB/s (touched bytes) at 1 "
                   "MI355X") if short else "chunked-prefill tokens/sec at 1 MI355X",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "new_tokens": spec["n_new"],
                   "prefix": spec["prefix"], "q_heads": spec["Hq"], "kv_heads": spec["Hkv"],
                   "idx_heads": spec["Hidx"], "head_dim": spec["D"], "idx_dim": spec["Di"],
                   "topk": spec["topk"], "init": spec["init"], "local": spec["local"],
                   "page": 128, "parallelism": "none"},
        "stages_ms": {"score_gemm": score_ms, "select": sel_ms, "attention": attn_ms},
        "mfma_tflops": {"score_gemm": score_tf, "attention": attn_tf,
                        "step": (f_score + f_attn + f_iv) / (ms * 1e-3) / 1e12},
        "mfma_frac": {"score_gemm": score_tf / peak, "attention": attn_tf / peak,
                      "step": (f_score + f_attn + f_iv) / (ms * 1e-3) / 1e12 / peak},
        "flops": {"score_gemm": f_score, "attention": f_attn, "index_value": f_iv},
        "ms_per_step_median": float(np.median(step_ms)),
        "wall_s_timed_region": t_wall,
        "roofline": roof,
        **device_info(dev),
    }
    if short:
        total_b = idx_b + kv_b + small_b
        res["hbm_gbps"] = total_b / (ms * 1e-3) / 1e9
        res["hbm_frac"] = res["hbm_gbps"] / HBM_PEAK_GBS
        res["touched_bytes"] = {"idx_keys": idx_b, "selected_kv_union": kv_b, "small": small_b}
    if headline and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(case, spec, args.cpu_seconds)
    return res


def measure_append(args, name, headline):
    """Paged append (msa_append_kv): T new tokens' K, V and index keys into
    the pools at seeded random slots, GB/s on the bytes it must move."""
    import torch

    import block_sparse_attention_score_amd as msa
    from synth import WORKLOAD_SEEDS, workload

    spec = workload(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device="cpu").manual_seed(WORKLOAD_SEEDS[name])
    T, Hkv, Hidx, D, Di = spec["T"], spec["Hkv"], spec["Hidx"], spec["D"], spec["Di"]
    P = (spec["pool_tokens"] + 127) // 128
    kv = spec["kv"]
    pool_dt = torch.uint8 if kv.startswith("fp8") else torch.bfloat16
    k_pool = torch.zeros((P, Hkv, 128, D), dtype=pool_dt, device=dev)
    v_pool = torch.zeros_like(k_pool)
    ik_pool = torch.zeros((P, Hidx, 128, Di), dtype=torch.bfloat16, device=dev)
    k_new = torch.randn((T, Hkv, D), generator=g).to(torch.bfloat16).to(dev)
    v_new = torch.randn((T, Hkv, D), generator=g).to(torch.bfloat16).to(dev)
    ik_new = torch.randn((T, Hidx, Di), generator=g).to(torch.bfloat16).to(dev)
    slots = torch.randperm(P * 128, generator=g)[:T].to(torch.int64).to(dev)
    cfg = msa.MsaConfig.from_spec(spec)
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def step():
        msa.append_kv(cfg, k_new, v_new, ik_new, slots, k_pool, v_pool, ik_pool)

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(i)
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ekv = elem_bytes(kv)
    moved = T * (2 * Hkv * D * 2 + Hidx * Di * 2 + 8) + T * (2 * Hkv * D * ekv + Hidx * Di * 2)
    gbps = moved / (ms * 1e-3) / 1e9
    res = {
        "metric": "paged KV append tokens/sec + achieved HBM GB/s at 1 MI355X",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": kv, "data": "synthetic",
        "config": {"workload": name, "new_tokens": T, "pool_pages": P,
                   "kv_heads": Hkv, "idx_heads": Hidx, "head_dim": D, "idx_dim": Di,
                   "kv_dtype": kv, "page": 128, "parallelism": "none"},
        "wall_s_timed_region": t_wall,
        "roofline": {"kernel": "append_kernel", "bound": "hbm", "achieved": gbps,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBS,
                     "traffic": None, "bytes_per_launch": moved, "ms_per_launch": ms},
        **device_info(dev),
    }
    return res


def chunk_touched_bytes(spec, seq_lens, cu, sel, cnt):
    """Algorithmic bytes of a short-chunk (multi-token decode) step: the index
    keys of every sequence once, the K/V of the union of its tokens' selected
    blocks (valid tokens), the queries, outputs, tables and selections."""
    Hq, Hkv, Hidx, D, Di = spec["Hq"], spec["Hkv"], spec["Hidx"], spec["D"], spec["Di"]
    ekv = elem_bytes(spec["kv"])
    gpi = Hkv // Hidx
    idx_b = kv_b = 0
    for b, L in enumerate(seq_lens.astype(np.int64)):
        idx_b += int(Hidx * L * Di * 2)
        for g in range(Hkv):
            blocks = set()
            for t in range(int(cu[b]), int(cu[b + 1])):
                blocks.update(int(j) for j in sel[t, g // gpi, : cnt[t, g // gpi]])
            kv_b += sum(min(128, int(L) - 128 * j) for j in blocks) * D * 2 * ekv
    T = int(cu[-1])
    nb = (seq_lens.astype(np.int64) + 127) // 128
    small = int(T * Hq * D * 2 * 2 + T * Hidx * Di * 2 + 4 * (nb.sum() + Hkv * cnt.sum()))
    return idx_b, kv_b, small


def cpu_baseline_prefill(case, spec, seconds):
    """The oracle on a bounded sample of prefill tokens (every sequence's new
    tokens, strided), as tokens/s."""
    import oracle
    from synth import host_view

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    inp = host_view(case)
    cu = case.cu_seqlens_q.cpu().numpy()
    L = case.seq_lens.cpu().numpy()
    done, t_used, stride = 0, 0.0, 64
    offset = 0
    while t_used < seconds and offset < stride:
        rows, pos = [], []
        for b in range(case.B):
            n = int(cu[b + 1] - cu[b])
            for i in range(offset, n, stride):
                rows.append(int(cu[b]) + i)
                pos.append((b, int(L[b]) - n + i))
        sub = dict(inp)
        sub["q"] = inp["q"][rows]
        sub["idx_q"] = inp["idx_q"][rows]
        sub["positions"] = pos
        t0 = time.perf_counter()
        oracle.sparse_attention(sub)
        t_used += time.perf_counter() - t0
        done += len(rows)
        offset += 1
    return dict(value=done / t_used, unit="tokens/s", cores=int(blas_threads),
                host_cpus=len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"{done} of {case.T} prefill tokens of {spec['name']} (every 64th "
                       f"token per sequence, all heads), {t_used:.1f} s of fp64 numpy")


if __name__ == "__main__":
    main()
