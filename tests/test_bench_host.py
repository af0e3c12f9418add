"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte counts
and the counter-record lookup that fills the roofline's `traffic`."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_bench_lines():
    # each tensor read or written once: x and y (2 bytes each), gamma and beta once, fp32
    # mean and rstd per row
    c5 = workloads.C5
    assert workloads.algorithmic_bytes(c5.op, c5.rows, c5.N, c5.elem_bytes, with_stats=True) == \
        2 * 4096 * 16384 * 2 + 2 * 16384 * 2 + 8 * 4096
    f = workloads.FUSED_8192
    # x, residual in; y, residual_out out; weight once; fp32 rstd per row
    assert workloads.algorithmic_bytes(f.op, f.rows, f.N, f.elem_bytes, with_stats=True) == \
        4 * 8192 * 4096 * 2 + 4096 * 2 + 4 * 8192


def test_counter_record_is_used_only_for_the_current_kernel_code(tmp_path, monkeypatch):
    rec = tmp_path / "counters.txt"
    rec.write_text(f"kernel_source_sha256_16: {bench.kernel_source_hash()}\n"
                   "ln_bf16_4096x16384 traffic_bytes_per_launch: 269288869\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(rec))
    assert bench.counter_traffic("ln_bf16_4096x16384") == 269288869.0
    assert bench.counter_traffic("fused_fp16_8192x4096") is None  # no record for it
    rec.write_text("kernel_source_sha256_16: 0000000000000000\n"
                   "ln_bf16_4096x16384 traffic_bytes_per_launch: 269288869\n")
    assert bench.counter_traffic("ln_bf16_4096x16384") is None  # recorded for other code
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.txt"))
    assert bench.counter_traffic("ln_bf16_4096x16384") is None


def test_kernel_fingerprint_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hpp", tmp_path / "b.hpp"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    b.write_text("/* two */\nint f(int x)\n{\n    return x + 1;\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(a)])
    ha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(b)])
    assert bench.kernel_source_hash() == ha
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != ha


def test_eager_fields():
    r = {"bytes": 8_000_000_000, "eager_ms_per_step": 2000.0}
    e = bench.eager_fields(r)
    assert e["value"] == 4.0 and e["pct_of_peak"] == 0.05 and e["ms_per_step"] == 2000.0


@pytest.mark.parametrize("key", ["graph", "eager"])
def test_timing_descriptions(key):
    assert "torch.cuda.synchronize()" in bench.TIMING[key]


def test_replay_spread():
    s = bench.spread({"repeats_ms": [0.047, 0.046, 0.0465, 0.0462, 0.048]})
    assert s["n"] == 5 and s["median_ms"] == 0.0465 and s["q1_ms"] == 0.0462 and s["q3_ms"] == 0.047
    assert bench.spread({"repeats_ms": None}) is None
