"""Host-side behaviour of bench.py that needs no GPU."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_measured_traffic_only_for_the_measured_sources(monkeypatch):
    """bench.py reports the stored scan traffic only while the scan's sources
    hash to the value it was measured on, and null otherwise."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "decode_b32_l32k_scan_hbm_traffic.json")) as f:
        stored = json.load(f)
    monkeypatch.setattr(bench, "source_hash", lambda names=None: stored["source_sha256"])
    assert bench.measured_traffic("decode_b32_l32k") == stored["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda names=None: "0" * 64)
    assert bench.measured_traffic("decode_b32_l32k") is None
    # a workload whose scan traffic was never measured reports none
    assert bench.measured_traffic("decode_b2_l2048") is None
