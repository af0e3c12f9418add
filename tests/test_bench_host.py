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


def _write_trace(d, marks, kernels):
    import csv as _csv

    with open(d / "trace_marker_api_trace.csv", "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Function", "Start_Timestamp", "End_Timestamp"])
        for name, a, b in marks:
            w.writerow([name, a, b])
    with open(d / "trace_kernel_trace.csv", "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Workgroup_Size_Y",
                    "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        for name, t, dur, wg, grid in kernels:
            w.writerow([name, t, t + dur, wg, 1, 1, grid, 1, 1])


def test_trace_by_range_attributes_dispatches_to_their_range(tmp_path):
    k = "void rn::rownorm_vec_kernel<2, 0, 8, 4, 1, true, 3, 62>(rn::Params)"
    kernels = [(k, 1000 + 10 * i, 5000 + i, 512, 512 * 512) for i in range(30)]  # in range a
    kernels += [(k, 3000 + 10 * i, 7000, 512, 512 * 1024) for i in range(25)]  # in range b, another grid
    kernels += [("void at::native::elementwise_kernel<128, 4>(int)", 1005, 100, 128, 128),  # torch: dropped
                (k, 2500, 100, 512, 512)]  # between the ranges: dropped
    _write_trace(tmp_path, [("bench:plan:s:a", 900, 2000), ("bench:plan:s:b", 2900, 4000),
                            ("other", 1000, 5000)], kernels)
    by = bench.trace_by_range(str(tmp_path))
    assert set(by) == {"plan:s:a", "plan:s:b"}
    (name, n, us, wg), = by["plan:s:a"]
    assert name == "rn::rownorm_vec_kernel<2, 0, 8, 4, 1, true, 3, 62>" and n == 30 and wg == 512
    assert us == pytest.approx(5.0145)  # median of 5000..5029 ns
    (name, n, us, wg), = by["plan:s:b"]
    assert n == 25 and wg == 1024 and us == pytest.approx(7.0)
    assert "plan:s:a" in bench.trace_summary(str(tmp_path))


def test_plan_sweep_report():
    cand = lambda label, us, W: {"label": label, "tuning": None, "us": us, "q1_us": us, "q3_us": us,  # noqa: E731
                                  "replays": 5, "pct_of_peak": 50.0, "vs_best": us / 10.0,
                                  "plan": {"variant": "workgroup", "waves_per_row": W, "chunks_per_lane": 4,
                                           "persistent": True}}
    sweep = {"shapes": {
        "s1": {"op": "ln", "dtype": "bf16", "rows": 4, "N": 8, "why": "w", "planner_vs_best": 1.1, "planner_rank": 2,
               "candidates": [cand("auto", 11.0, 2), cand("W4xV2 persistent", 10.0, 4), cand("x", 30.0, 1)]},
        "s2": {"op": "ln", "dtype": "bf16", "rows": 4, "N": 8, "why": "w", "planner_vs_best": 1.0, "planner_rank": 1,
               "candidates": [cand("auto", 10.0, 2)]}}}
    md = bench.plan_sweep_report(sweep)
    assert "geometric mean 1.049x, worst 1.100x" in md
    assert "**planner** (W2xV4 persistent, grid rule)" in md
    # top=1 keeps the fastest, the planner's and the slowest
    md1 = bench.plan_sweep_report(sweep, top=1)
    assert md1.count("| x |") == 1 and md1.count("W4xV2 persistent") == 1


def test_traffic_summary_scales_and_attributes(tmp_path, monkeypatch):
    import csv as _csv

    def counters(d, prefix, rows):
        d.mkdir()
        with open(d / f"{prefix}_counter_collection.csv", "w", newline="") as f:
            w = _csv.writer(f)
            w.writerow(["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Value"])
            w.writerows(rows)

    copy = "void (anonymous namespace)::stream_copy_kernel<512, 2, true>(char const*, char*, long)"
    k = "void rn::rownorm_vec_kernel<2, 0, 8, 4, 1, true, 3, 62>(rn::Params)"
    # the copy reads 262144 KiB and writes 262144 KiB: FETCH_SIZE counts half, WRITE_SIZE all
    counters(tmp_path / "cf", "cal", [[copy, 1024, 512, 131072.0]] * 3)
    counters(tmp_path / "cw", "cal", [[copy, 1024, 512, 262144.0]] * 3)
    counters(tmp_path / "pf", "pmc", [[k, 512 * 512, 512, 65536.0]] * 5)
    counters(tmp_path / "pw", "pmc", [[k, 512 * 512, 512, 131072.0]] * 5)
    tr = tmp_path / "tr"
    tr.mkdir()
    _write_trace(tr, [("bench:C5_ln_bf16_4096x16384:cold", 0, 10 ** 6)],
                 [(k, 10 + i, 45000, 512, 512 * 512) for i in range(30)])
    out = bench.traffic_summary(str(tmp_path / "pf"), str(tmp_path / "pw"), str(tmp_path / "cf"),
                                str(tmp_path / "cw"), str(tr))
    # 65536 KiB * 2 + 131072 KiB = 262144 KiB per launch, recorded under the headline's key
    assert "ln_bf16_4096x16384 traffic_bytes_per_launch: 268435456" in out
    assert f"kernel_source_sha256_16: {bench.kernel_source_hash()}" in out
    rec = tmp_path / "rec.txt"
    rec.write_text(out)
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(rec))
    assert bench.counter_traffic("ln_bf16_4096x16384") == 268435456
