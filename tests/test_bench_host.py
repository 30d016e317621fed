"""Host-side pieces of bench.py (no GPU): argument handling, the workload string, the kept-flop
count and the traffic lookup, so that a slip in them shows here rather than in a GPU run."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_workload_name():
    assert bench.workload_name("720p", 0, None, 1, 40, 75600, 128, 128, 0.15, 89, 591) == (
        "720p: B=1 H=40 S=75600 D=128 block=128 keep_ratio=0.15 (89 of 591 key blocks kept)")
    name = bench.workload_name("720p", 5, 7, 1, 5, 75600, 128, 128, 0.15, 89, 591)
    assert name.startswith("720p (first 5 heads: one rank's share) (seed 7): B=1 H=5 ")


def test_kept_flops_counts_partial_blocks():
    # S = 300, block 128: blocks of 128, 128 and 44 tokens; one row keeps {0, 2}, one keeps {2}
    rp = np.array([0, 2, 3, 3], np.int32)
    ci = np.array([0, 2, 2], np.int32)
    # row 0 (128 queries): 128*(128 + 44); row 1 (128 queries): 128*44; row 2 (44 queries): none
    assert bench.kept_flops(rp, ci, 300, 128) == 128 * (128 + 44) + 128 * 44


def test_traffic_lookup_needs_the_current_kernel():
    assert bench.traffic_from_profile("0" * 64) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help_lists_the_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for opt in ("--all-configs", "--heads", "--mfma-peak", "--seed", "--sweep"):
        assert opt in r.stdout


def test_cpu_baseline_on_a_workload_smaller_than_the_sample():
    import gen
    q, k, v, cfg = gen.make_config("tiny")
    r = bench.cpu_baseline(q, k, v, cfg, 8192)
    assert r["kind"] == "oracle" and r["value"] > 0 and "2048 of 2048" in r["sample"]
