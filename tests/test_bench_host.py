"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the roofline
accounting and the committed profile lookup."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sketch_attention_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_accounting_of_the_long_workload():
    # 4 users x 100000 rows, d = 128, k = 256, bf16: 4kd FLOP and 2d bytes per row, plus the sketches
    assert bench.algorithmic_flops(256, 128, 400000) == 4 * 256 * 128 * 400000
    assert bench.algorithmic_bytes(400000, 4, 256, 128, 2) == 400000 * 128 * 2 + 4 * 4 * 256 * 128
    ratio = bench.algorithmic_flops(256, 128, 400000) / bench.algorithmic_bytes(400000, 4, 256, 128, 2)
    assert 500 < ratio < 512  # above the bf16 ridge (about 312 FLOP/B): the matrix cores bound it


def test_profile_lookup_requires_the_current_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    f = tmp_path / "sa_fused_long_hbm_bytes.md"
    f.write_text(f"kernel_source_sha256: {bench.kernel_source_hash('bf16', 128)}\ntraffic_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("long", "bf16", 128) == 123456.0
    f.write_text("kernel_source_sha256: 0000\ntraffic_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("long", "bf16", 128) is None
    assert bench.measured_traffic("ragged", "bf16", 128) is None  # no summary for that workload


def test_kernel_hash_is_deterministic_and_covers_the_streamed_pass():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 64


def test_stack_weights_are_seeded():
    a = W.make_stack_layers(d=64, d_ff=128, layers=2, dtype="bf16", seed=3)
    b = W.make_stack_layers(d=64, d_ff=128, layers=2, dtype="bf16", seed=3)
    assert all(np.array_equal(x[k], y[k]) for x, y in zip(a, b) for k in x)
    assert a[0]["W_Q"].dtype == np.float32 and a[0]["ffn_down"].shape == (128, 64)


@pytest.mark.parametrize("flags", [["--actions", "--grad"], ["--actions", "--layers", "2"], ["--grad", "--norm", "history"],
                                   ["--norm", "history", "--layers", "2"]])
def test_conflicting_modes_are_refused_before_any_gpu_work(flags):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "only" in r.stderr and r.stdout == ""


def test_kernel_timing_pass_is_long_enough():
    # the driver's short runs (e.g. 20 steps) still average the kernel durations over >= 50 launches
    assert bench.kernel_timing_steps(20) == 50
    assert bench.kernel_timing_steps(400) == 400
    assert bench.timing_period(20) == 1 and bench.timing_period(400) == 8  # the secondary modes


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model() != ""


def test_roofline_kernel_label_follows_the_planner():
    # the kernel the bench line names for each workload shape (make_plan's rule)
    assert bench.fused_kernel_name("bf16", 128, 256) == "sa_wide_kernel"
    assert bench.fused_kernel_name("bf16", 128, 256, "history") == "sa_stream_kernel"
    assert bench.fused_kernel_name("bf16", 128, 1024) == "sa_stream32_kernel"
    assert bench.fused_kernel_name("bf16", 128, 64) == "sa_stream_kernel"
    assert bench.fused_kernel_name("bf16", 128, 128) == "sa_stream_kernel"
    assert bench.fused_kernel_name("bf16", 64, 1024) == "sa_stream_kernel"
    assert bench.fused_kernel_name("f32", 64, 16) == "sa_fused_kernel"
    assert bench.fused_kernel_name("bf16", 128, 32) == "sa_fused_kernel"
