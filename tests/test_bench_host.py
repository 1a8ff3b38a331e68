"""bench.py on the host: the script imports without a GPU (no syntax or
import errors reach the measured run), asks for one GPU, and reads the
committed HBM-counter summaries for the forward."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_imports_and_constants():
    import bench
    assert bench.BWD_WARMUP >= 1
    assert bench.PEAK_HBM_GBPS == 8000.0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_traffic_matches_the_forward_source():
    import bench
    # the committed summary was taken from the current attn.hip, so its traffic figure is used
    assert bench.counter_traffic("sft") is not None
