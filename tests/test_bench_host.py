"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the roofline's
work accounting and the staleness rule of the committed traffic figures."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_alu_peak_is_the_fp32_vector_rate_in_lane_operations():
    # 157.3 TFLOP/s counts an FMA as two flops
    assert abs(bench.ALU_PEAK * 2 - 157.3e12) / 157.3e12 < 1e-3


def test_blocked_order_flush_work():
    # one PS(mu) add (add + 3-instruction rounding) per run; none when the
    # order is sequential (block 0 or 1, or a run covering the whole dot)
    assert bench.run_flush_ops(64, 0) == 0
    assert bench.run_flush_ops(64, 1) == 0
    assert bench.run_flush_ops(64, 64) == 0
    assert bench.run_flush_ops(64, 16) == 16
    assert bench.run_flush_ops(100, 8) == 4 * 13


def test_traffic_entries_follow_the_kernel_sources():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        tab = json.load(f)
    for key, ent in tab.items():
        kernel, workload = key.split("/", 1)
        got = bench.load_traffic(kernel, workload)
        if ent["source_sha"] == bench.kernel_source_sha(kernel):
            assert got == ent["bytes_per_launch"], key
        else:   # measured on other sources: reported as unknown
            assert got is None, key
    assert bench.load_traffic("ps_scores_kernel", "no_such_workload") is None
