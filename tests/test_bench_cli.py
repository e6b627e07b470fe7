"""Host-side checks of bench.py's contract (no GPU): one GPU only, and the HBM traffic figure
is reported only for the workload and kernel source the counters were taken on."""
import argparse
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_profiled_source_and_workload():
    src = os.path.join(ROOT, "sparse_attention_token_idx_amd", "csrc", "prefill.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    ok = argparse.Namespace(T=65536, topk=2048)
    want = bench.TRAFFIC_FILTER_T65536["bytes"] if h == bench.TRAFFIC_FILTER_T65536["source_sha256_prefix"] else None
    assert bench.filter_traffic(ok) == want
    assert bench.filter_traffic(argparse.Namespace(T=8192, topk=2048)) is None
    assert bench.filter_traffic(argparse.Namespace(T=65536, topk=512)) is None


def test_stats_median_min_mean():
    s = bench.stats([3.0, 1.0, 2.0, 10.0])
    assert s == {"median": 2.5, "min": 1.0, "mean": 4.0}
