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


def test_counter_traffic_only_from_the_current_source(tmp_path):
    """A counter summary is used only while the forward's source still hashes
    to the one it records; otherwise the line reports traffic as null."""
    import hashlib

    import bench
    src_dir = tmp_path / "packed_varlen_causal_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "attn.hip"
    src.write_bytes(b"// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    summary = tmp_path / "profiles" / "attn_fwd_longctx_hbm_counters.md"
    summary.write_text(f"# summary\n\nattention_traffic_bytes_per_launch: 1234.0\nattn_source_sha256_prefix: {sha}\n")
    assert bench.counter_traffic("longctx", root=str(tmp_path)) == 1234.0
    assert bench.counter_traffic("sft", root=str(tmp_path)) is None
    src.write_bytes(b"// changed kernel source\n")
    assert bench.counter_traffic("longctx", root=str(tmp_path)) is None


def test_headline_is_the_long_context_buffer():
    """The default workload is the long-context buffer (131,072 tokens, 32
    heads, d = 128), the configuration of the 40%-of-peak target."""
    import bench
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="longctx")' in src
    from workloads import make_workload
    w = make_workload("longctx")
    assert (w.total_tokens, w.heads, w.head_dim) == (131072, 32, 128)
    assert bench.useful_flops(w.lengths, w.is_pad, w.heads, w.head_dim) > 1e13


def test_roofline_block_picks_the_binding_roof():
    import types

    import bench
    x = types.SimpleNamespace(T=131072, H=32, D=128, flops=1.26e13)
    r = bench.roofline(x, 12.6, "k")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - 1.26e13 / 12.6e-3 / 1e12 / 2500.0) < 1e-4
    y = types.SimpleNamespace(T=65536, H=32, D=128, flops=2.1146e11)
    r = bench.roofline(y, 0.5, "k", traffic=2.2e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - 4 * 65536 * 32 * 128 * 2 / 0.5e-3 / 1e9) < 0.1
    assert r["traffic_over_algorithmic_bytes"] == round(2.2e9 / (4 * 65536 * 32 * 128 * 2), 3)
