"""The benchmark's command line on a host without a GPU: it refuses more
than one GPU with a message, and its helpers compute what they state."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_quantile_and_algorithmic_counts():
    import bench
    from workloads import WORKLOADS
    assert bench.quantile([3.0, 1.0, 2.0], 0.5) == 2.0
    assert bench.quantile([1.0, 2.0], 0.25) == pytest.approx(1.25)
    assert bench.quantile([5.0], 0.8) == 5.0
    w = WORKLOADS["same_device"]
    # x + out (fp32) + B + C + dt + A + final state, written out by hand
    T, H, P, N, G = 4 * 2048, 16, 64, 128, 4
    want = T * H * P * 8 + 2 * T * G * N * 4 + 4 * T * H + 4 * H + 4 * 4 * H * P * N
    assert bench.algorithmic_bytes(w) == want
    nc = 2048 // 128
    assert bench.algorithmic_flops(w) == 2 * 4 * nc * (G * 128 * 128 * N + H * 128 * 128 * P
                                                       + 2 * H * 128 * N * P)


def test_processes_run_children_and_stop_on_a_failed_one():
    # without a GPU the first child exits 2 ("needs a GPU"); the parent stops
    # there with that code and prints no JSON line
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--processes", "3",
                        "--steps", "1"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 2
    assert "process 1 of 3" in r.stderr and "process 1 failed" in r.stderr
    assert "process 2 of 3" not in r.stderr
    assert r.stdout.strip() == ""
