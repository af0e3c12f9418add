#!/usr/bin/env python3
"""Benchmark of the row-wise normalization hot path on one MI355X.

One step = one LayerNorm forward (y, mean, rstd) over the 4096 x 16384 bf16 workload, the
largest configuration and the one the bandwidth target applies to (rows * N = 64M >= 8M).
The same measurement is also taken for fused residual-add + RMSNorm at 8192 x 4096 fp16
(32M elements) and reported in the same JSON line under "fused_add_rms_norm", and, under
"more", for fused residual-add + LayerNorm (8192 x 4096 bf16), softmax (8192 x 4096 fp32),
the LayerNorm backward (4096 x 16384 bf16: dx, dgamma, dbeta), the RMSNorm backward
(8192 x 4096 fp16: dx, dweight), ragged LayerNorm rows (16384 x 4095 bf16), split rows
(LayerNorm 1024 x 65536 fp32), a vocabulary-sized softmax (1024 x 50257 fp32, byte-addressed
rows) and the split-row LayerNorm backward (1024 x 65536 bf16); under "scale_up_sweep", fused add + RMSNorm at
N = 4096 over 2048 / 8192 / 32768 rows (fp16 and bf16), LayerNorm bf16 at N = 4096 over 2048 / 4096 / 8192 rows, and the
headline workload with a hot cache; under "configs", every listed configuration (cold and
hot, events and graph replay, next to the oracle's host throughput). Small launches (tens of microseconds) are shorter than
the Python binding's per-call host time, so the sweep also replays its launches from a HIP
graph ("graph_ms": device time per launch without host gaps).

Cold cache: inputs and outputs rotate through enough buffer sets (at least four, at least
1 GiB per cycle) that each launch touches memory the previous launches have pushed out of
L2 (8 x 4 MiB) and the 256 MiB memory-side cache. Inputs are resident in HBM before the timed region starts.

Timed region: the workload's own launches for about 300 ms first (the GPU has been idle
during the host-side set-up, and its first milliseconds of work run slower), W warmup steps
untimed, then exactly K steps launched eagerly from Python, bracketed by
torch.cuda.synchronize() ("eager": wall time over K), then the same K steps captured into
one HIP graph, replayed once untimed and then at least five times and for at least 200 ms
of device time (--replay-ms), each replay between torch.cuda.synchronize() calls:
ms_per_step is the median of the replays' wall time over K (the eager time when no graph
can be captured; "timing" says which). A graph is how a serving or training loop runs a
fixed sequence of launches: each step still launches its kernel on its own rotating
buffers; only the per-call Python and dispatch overhead between steps (about 2 us per
launch here) is gone. Two HIP events recorded on the launch stream (torch's current
stream, which the binding passes to the C ABI) around each timed replay give the
per-launch kernel duration used for the roofline (their median); rocprofv3's kernel
durations agree with it. "replays" gives their spread (median and quartiles of the
per-step device time).

Ceiling: a hand-written streaming copy kernel (libstreamprobe.so, include/stream_probe.h)
timed the same way at the traffic of LayerNorm bf16 at 8M elements, fused add + RMSNorm at
8M elements and the 4096 x 16384 LayerNorm ("ceiling"); the roofline and the 8M-element
sweep points also report their fraction of that measured ceiling. The CPU baseline runs
last, after every GPU line, so that its seconds of host-only work do not precede a timed
region.

value = algorithmic bytes per step / ms_per_step (GB/s, 1 GB = 1e9 B). Algorithmic bytes:
LayerNorm 2*rows*N*s + 2*N*s + 8*rows; fused 4*rows*N*s + N*s + 4*rows (with rstd); fused
LayerNorm 4*rows*N*s + 2*N*s + 8*rows; softmax 2*rows*N*s; LayerNorm backward
3*rows*N*s + 3*N*s + 8*rows; RMSNorm backward 3*rows*N*s + 2*N*s + 4*rows. (The backward's
fp32 partial column rows are not algorithmic bytes: they count against it.)

The CPU baseline times the fp64 oracle (oracle/) on the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--cache cold|hot] [--replay-ms MS]
       python bench.py --ceiling-sweep      (every geometry of the copy kernel at the ceiling sizes)
       python bench.py --copy-calibration   (plain copy of known size, for counter scaling)
       python bench.py --plan-sweep --steps 20 --replay-ms 40   (automatic launch plans against
                                            every built alternative, JSON)
       python bench.py --plan-sweep-report SWEEP.json [--trace DIR]   (its markdown tables)
       python bench.py --trace-summary DIR  (kernels per roctx range of a rocprofv3 trace of this script)
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of MI355X peak) + rows/s, LayerNorm & fused add+RMSNorm"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published peak
COLD_FOOTPRINT = 1 << 30  # bytes each buffer set cycle must exceed (L2 + 256 MiB MALL, with margin)
MIN_COLD_SETS = 4  # buffer sets a cold-cache line rotates through at least
KERNEL_SRCS = [os.path.join(ROOT, "row_wise_normalization_fp32_amd", "csrc", f)
               for f in ("rownorm_kernels.hpp", "rownorm_backward.hpp", "rownorm_capi.cpp")]  # kernels + launch plan
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Fingerprint of the code that decides the kernel: the sources with comments and
    whitespace removed, so that only a change of the code itself invalidates a counter
    record."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload_key: str):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a copy
    kernel), if recorded for the current kernel source; else None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^{re.escape(workload_key)}\s+traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    return float(m.group(1)) if m else None


def make_sets(w, nsets, dev):
    import torch

    import row_wise_normalization_fp32_amd as rn
    import workloads

    base = workloads.make_inputs(w)
    sets = []
    for i in range(nsets):
        s = {}
        for k, v in base.items():
            if k in ("gamma", "beta", "weight"):
                s[k] = sets[0][k] if sets else v.to(dev)
            else:
                # distinct buffers with the workload's values (a rolled copy per set)
                s[k] = torch.roll(v, shifts=i, dims=0).to(dev) if i else v.to(dev)
        s["rstd"] = torch.empty(w.rows, dtype=torch.float32, device=dev)
        s["mean"] = torch.empty(w.rows, dtype=torch.float32, device=dev)
        if w.op in ("ln_bwd", "rms_bwd"):
            # the forward statistics the backward consumes (computed once, outside timing)
            if w.op == "ln_bwd":
                rn.ln_forward(s["x"], None, None, w.eps, mean=s["mean"], rstd=s["rstd"])
            else:
                rn.rms_norm(s["x"], None, w.eps, rstd=s["rstd"])
            s["dx"] = torch.empty_like(s["x"])
            s["ws"] = torch.empty(rn.backward_workspace_bytes("ln" if w.op == "ln_bwd" else "rms", w.rows, w.N),
                                  dtype=torch.uint8, device=dev)
        else:
            s["y"] = torch.empty_like(s["x"])
        if w.op in ("fused_add_rms", "fused_add_ln"):
            s["residual_out"] = torch.empty_like(s["x"])
        sets.append(s)
    return sets


def kernel_name(w, plan):
    """The kernel instance a workload's launch runs, as rocprofv3 lists it (template arguments:
    dtype, op, waves per row, chunks per lane, row groups per workgroup, exact, affine, flags)."""
    if w.op in ("ln_bwd", "rms_bwd"):
        if plan["variant"] == "wide":
            return (f"rn::rownorm_bwd_wide_clear_kernel + rn::rownorm_bwd_wide_onepass_kernel ({w.dtype}, {w.op}, "
                    f"8192-element segments, 512 lanes each, at most {plan['grid_blocks']} row blocks) "
                    f"+ rn::rownorm_bwd_cols_kernel")
        k = "rownorm_bwd_vec_kernel" if plan["variant"] == "workgroup" else "rownorm_bwd_elem_kernel"
        return (f"rn::{k} ({w.dtype}, {w.op}, W={plan['waves_per_row']} waves per row, V={plan['chunks_per_lane']}, "
                f"{plan['rows_per_block']} row group(s) per workgroup) + rn::rownorm_bwd_cols_kernel")
    if plan["variant"] == "general":
        return f"rn::rownorm_general_kernel ({w.dtype}, {w.op})"
    if plan["variant"] == "wide":
        # the bench passes the full workspace and writes out of place: the one-pass form
        return (f"rn::rownorm_wide_clear_kernel + rn::rownorm_wide_onepass_kernel ({w.dtype}, {w.op}, 32 KiB "
                f"segments, one 512-lane workgroup per (row block, segment) ticket, {plan['grid_blocks']} row "
                f"segments, x read once)")
    if plan["variant"] == "wide_element":
        return (f"rn::rownorm_wide_elem_stats_kernel + rn::rownorm_wide_elem_norm_kernel ({w.dtype}, {w.op}, one "
                f"512-lane workgroup per row segment, {plan['grid_blocks']} segments)")
    mode = "persistent" if plan["persistent"] else "grid per row"
    if plan.get("ragged"):
        mode += ", byte-addressed rows"
    if plan["variant"] == "element":
        k = "rownorm_pair_kernel" if plan.get("pairs") else "rownorm_elem_kernel"
    else:
        k = "rownorm_vec_kernel"
    return (f"rn::{k} ({w.dtype}, {w.op}, W={plan['waves_per_row']} waves per row, "
            f"V={plan['chunks_per_lane']} per lane, {plan['rows_per_block']} row group(s) per workgroup, {mode})")


def launch(rn, w, s, tuning=None):
    """One call of workload `w` on buffer set `s` (forward ops: with an optional tuning, whose
    "variant" key, if any, forces a kernel variant)."""
    kw = {}
    if tuning is not None:
        t = dict(tuning)
        if "variant" in t:
            kw["variant"] = t.pop("variant")
        if t:
            kw["tuning"] = t
    if w.op == "ln":
        rn.ln_forward(s["x"], s.get("gamma"), s.get("beta"), w.eps, out=s["y"], mean=s["mean"], rstd=s["rstd"], **kw)
    elif w.op == "rms":
        rn.rms_norm(s["x"], s.get("weight"), w.eps, out=s["y"], rstd=s["rstd"], **kw)
    elif w.op == "fused_add_rms":
        rn.fused_add_rms_norm(s["x"], s["residual"], s.get("weight"), w.eps, out=s["y"],
                              residual_out=s["residual_out"], rstd=s["rstd"], **kw)
    elif w.op == "fused_add_ln":
        rn.fused_add_layer_norm(s["x"], s["residual"], s.get("gamma"), s.get("beta"), w.eps, out=s["y"],
                                residual_out=s["residual_out"], mean=s["mean"], rstd=s["rstd"], **kw)
    elif w.op == "softmax":
        rn.softmax_forward(s["x"], out=s["y"], **kw)
    elif w.op == "ln_bwd":
        rn.ln_backward(s["dy"], s["x"], s["mean"], s["rstd"], s.get("gamma"), dx=s["dx"], workspace=s["ws"])
    elif w.op == "rms_bwd":
        rn.rms_norm_backward(s["dy"], s["x"], s["rstd"], s.get("weight"), dx=s["dx"], workspace=s["ws"])
    else:
        raise ValueError(w.op)


SET_TENSORS = {"ln": 2, "rms": 2, "softmax": 2, "fused_add_rms": 4, "fused_add_ln": 4, "ln_bwd": 3, "rms_bwd": 3}


REPEATS = 5  # timed replays of a graph at least ...
MIN_REPLAY_MS = 200.0  # ... and until they add up to this much device time (at most MAX_REPLAYS)
MAX_REPLAYS = 400


def spread(r):
    """Median and quartiles of the per-step device time over the timed replays."""
    reps = sorted(r.get("repeats_ms") or [])
    if not reps:
        return None
    q = lambda f: reps[min(len(reps) - 1, int(round(f * (len(reps) - 1))))]  # noqa: E731
    return {"n": len(reps), "median_ms": round(q(0.5), 5), "q1_ms": round(q(0.25), 5), "q3_ms": round(q(0.75), 5),
            "what": f"{len(reps)} timed replays of one HIP graph of the K steps, HIP events around each"}


def replay_count(first_replay_ms: float) -> int:
    """Timed replays: at least REPEATS, and enough to cover MIN_REPLAY_MS of device time (a
    replay of a few short steps lasts about a millisecond, too short for a stable median),
    at most MAX_REPLAYS."""
    if first_replay_ms <= 0:
        return REPEATS
    return int(max(REPEATS, min(MAX_REPLAYS, math.ceil(MIN_REPLAY_MS / first_replay_ms))))


def graph_time_fn(step, steps):
    """`steps` calls of step(i) captured into one HIP graph, replayed once to warm up, then
    timed replays (replay_count), each bracketed by torch.cuda.synchronize() (wall clock) and
    by two HIP events on the launch stream. Returns the medians per step ({"wall_ms",
    "event_ms"}) and every replay's per-step event time ("repeats_ms"), or None if the
    capture fails."""
    import torch

    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        n = replay_count(a.elapsed_time(b))
        walls, events = [], []
        for _ in range(n):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - t0) * 1e3 / steps)
            events.append(a.elapsed_time(b) / steps)
        del g
        med = lambda v: sorted(v)[len(v) // 2]  # noqa: E731
        return {"wall_ms": med(walls), "event_ms": med(events), "repeats_ms": events, "walls_ms": walls}
    except Exception as e:  # capture not possible here: report without it
        log(f"[bench] graph timing unavailable: {e}")
        return None


def graph_time(rn, w, sets, steps):
    """The K steps of workload `w`, rotating over its buffer sets, as a replayed HIP graph."""
    return graph_time_fn(lambda i: launch(rn, w, sets[i % len(sets)]), steps)


TIMING = {
    "graph": "K steps captured in one HIP graph; median over the timed replays (at least 5, and at least "
             "200 ms of device time), each timed by wall clock between torch.cuda.synchronize() calls (after "
             "the workload's own launches for about 300 ms, an untimed eager pass and an untimed replay)",
    "eager": "K eager launches timed by wall clock between torch.cuda.synchronize() calls",
}


def eager_fields(r):
    """The same K steps launched eagerly from Python (one binding call each)."""
    v = r["bytes"] / (r["eager_ms_per_step"] * 1e-3) / 1e9
    return {"ms_per_step": round(r["eager_ms_per_step"], 5), "value": round(v, 2),
            "pct_of_peak": round(100.0 * v / PEAK_HBM_GBS, 2)}


def kernel_time(r):
    """Per-launch device time for the roofline: from the replays of a HIP graph holding the
    K timed launches (median of the HIP events around each replay, on the launch stream),
    which leave out the dispatch gaps of eager back-to-back launches (≈2 µs each here, which
    rocprofv3's kernel durations also leave out); the eager stream events when no graph
    could be captured."""
    if r.get("graph_ms"):
        n = len(r.get("repeats_ms") or []) or REPEATS
        return r["graph_ms"], (f"median over {n} replays of a HIP graph of the K timed launches, "
                               "HIP events around each")
    return r["kernel_ms"], "HIP events around the K eager launches (no graph capture)"


PRIME_MS = 300.0


def prime_gpu(step, ms=None):
    """Runs the workload's own launches (step(i), eagerly) for about `ms` before a
    measurement. After the host-side set-up of a workload (or the CPU baseline) the GPU
    has been idle, and its first milliseconds of work run slower (measured: C5 LayerNorm
    launches at 47-51 us, then a steady 46.3 us; a 50 ms prime of plain copies still left
    the timed replays of a short run 4% slower than the same kernel later in the run). The
    launches write only the workload's own output buffers."""
    import torch

    ms = PRIME_MS if ms is None else min(ms, PRIME_MS)
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()


class line_marker:
    """A roctx range (torch.cuda.nvtx) around one bench line, named "bench:<line>", so that a
    rocprofv3 --marker-trace run can attribute each kernel dispatch to its line."""

    def __init__(self, name):
        self.name = name

    def __enter__(self):
        import torch

        torch.cuda.nvtx.range_push(f"bench:{self.name}")

    def __exit__(self, *exc):
        import torch

        torch.cuda.synchronize()
        torch.cuda.nvtx.range_pop()


def measure(w, steps, warmup, cache, dev, graph=True):
    with line_marker(f"{w.name}:{cache}"):
        return _measure(w, steps, warmup, cache, dev, graph)


def _measure(w, steps, warmup, cache, dev, graph=True):
    import torch

    import row_wise_normalization_fp32_amd as rn
    import workloads

    nbytes = workloads.algorithmic_bytes(w.op, w.rows, w.N, w.elem_bytes, with_stats=True)
    set_bytes = SET_TENSORS[w.op] * w.rows * w.N * w.elem_bytes
    nsets = 1 if cache == "hot" else max(MIN_COLD_SETS, min(64, math.ceil(COLD_FOOTPRINT / set_bytes)))
    log(f"[bench] {w.name}: {nsets} buffer set(s), {nbytes} algorithmic bytes per launch")
    sets = make_sets(w, nsets, dev)
    torch.cuda.synchronize()
    prime_gpu(lambda i: launch(rn, w, sets[i % nsets]))
    for i in range(warmup):
        launch(rn, w, sets[i % nsets])
    # Timed region: exactly `steps` steps, nothing else enqueued between them, bracketed by
    # torch.cuda.synchronize() (wall clock) and by two HIP events on the stream the kernels
    # run on (torch's current stream, which the binding passes to the C ABI): the device
    # time per step, the kernel duration used for the roofline.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        launch(rn, w, sets[(warmup + i) % nsets])
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms = wall * 1e3 / steps
    kernel_ms = ev0.elapsed_time(ev1) / steps
    gt = graph_time(rn, w, sets, steps) if graph else None
    graph_ms = gt["event_ms"] if gt else None
    # the steps as one replayed HIP graph when it can be captured, else the eager launches
    ms_per_step = gt["wall_ms"] if gt else eager_ms
    s0 = sets[0]
    td = workloads.TORCH_DTYPES[w.dtype]
    if w.op in ("ln_bwd", "rms_bwd"):
        # the plan of the timed call (host only): it passes a workspace, which split rows need
        st, info = rn.plan_backward("ln" if w.op == "ln_bwd" else "rms", w.rows, w.N, td,
                                    ptrs={"workspace": s0["ws"].data_ptr()})
        info["persistent"] = True
    else:
        ptrs = {k: s0[k].data_ptr() for k in ("x", "residual", "gamma", "beta", "weight", "y", "residual_out", "mean",
                                              "rstd") if k in s0}
        if "weight" in ptrs:
            ptrs["gamma"] = ptrs.pop("weight")
        if w.op == "softmax":
            ptrs.pop("mean", None)
            ptrs.pop("rstd", None)
        st, info = rn.plan(w.op, w.rows, w.N, td, ptrs=ptrs, eps=w.eps,
                           workspace_bytes=rn.forward_workspace_bytes(w.op, w.rows, w.N, td))
    del sets
    torch.cuda.empty_cache()
    return {
        "bytes": nbytes, "ms_per_step": ms_per_step, "timing": "graph" if gt else "eager",
        "eager_ms_per_step": eager_ms, "kernel_ms": kernel_ms, "graph_ms": graph_ms,
        "repeats_ms": gt["repeats_ms"] if gt else None,
        "nsets": nsets, "plan": info,
    }


def cpu_baseline(w, seconds, single_thread=False):
    """The oracle on `w` over about `seconds` of host time (median pass)."""
    import oracle
    import workloads

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    inp = workloads.make_inputs(w)
    nbytes = workloads.algorithmic_bytes(w.op, w.rows, w.N, w.elem_bytes, with_stats=True)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if w.op == "ln":
            oracle.layer_norm(inp["x"], inp.get("gamma"), inp.get("beta"), w.eps, threads=threads)
        elif w.op == "rms":
            oracle.rms_norm(inp["x"], inp.get("weight"), w.eps, threads=threads)
        else:
            oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp.get("weight"), w.eps, threads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= seconds or len(times) >= 2000:
            break
    med = sorted(times)[len(times) // 2]
    out = {
        "value": round(nbytes / med / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "rows_per_s": round(w.rows / med, 1),
        "sample": f"full {w.rows}x{w.N} {w.dtype} workload, {len(times)} passes over {sum(times):.1f} s, median pass",
    }
    if single_thread and threads > 1:
        # the same oracle on one host thread, over the first rows of the workload (about a
        # quarter of the multi-threaded budget), scaled to the whole workload's rows/s
        sub = {k: (v[: max(1, w.rows // 8)] if v.dim() == 2 else v) for k, v in inp.items()}
        rows1 = sub["x"].shape[0]
        t1 = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < seconds / 4 and len(t1) < 200:
            t0 = time.perf_counter()
            if w.op == "ln":
                oracle.layer_norm(sub["x"], sub.get("gamma"), sub.get("beta"), w.eps, threads=1)
            elif w.op == "rms":
                oracle.rms_norm(sub["x"], sub.get("weight"), w.eps, threads=1)
            else:
                oracle.fused_add_rms_norm(sub["x"], sub["residual"], sub.get("weight"), w.eps, threads=1)
            t1.append(time.perf_counter() - t0)
        m1 = sorted(t1)[len(t1) // 2]
        b1 = workloads.algorithmic_bytes(w.op, rows1, w.N, w.elem_bytes, with_stats=True)
        out["single_thread"] = {"value": round(b1 / m1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "rows_per_s": round(rows1 / m1, 1),
                                "sample": f"first {rows1} rows, {len(t1)} passes, median pass"}
    return out


PROBE_PATH = os.path.join(ROOT, "row_wise_normalization_fp32_amd", "libstreamprobe.so")
# Geometry of the ceiling copy kernel (include/stream_probe.h) at each size (key: bytes read
# per launch): 16-byte chunks per lane, lanes per workgroup, workgroups per CU (0: one
# workgroup per tile; k > 0: k per CU, looping over the tiles), non-temporal accesses. Each
# is the fastest of the 64 geometries `python bench.py --ceiling-sweep` times on MI355X
# (profiles/stream_ceiling_sweep.md).
CEILING_GEOM = {
    16 << 20: {"chunks_per_lane": 4, "block_threads": 256, "per_cu": 0, "nontemporal": 1},
    32 << 20: {"chunks_per_lane": 1, "block_threads": 256, "per_cu": 4, "nontemporal": 1},
    128 << 20: {"chunks_per_lane": 2, "block_threads": 512, "per_cu": 0, "nontemporal": 1},
}
# Traffic sizes (bytes read = bytes written) of the ceiling: LayerNorm bf16 at 8M elements
# (x 16 MiB), fused add + RMSNorm at 8M (x + residual 32 MiB), and the 4096 x 16384 bf16
# LayerNorm (x 128 MiB).
CEILING_READ_BYTES = tuple(sorted(CEILING_GEOM))


def probe_lib():
    import ctypes

    if not os.path.exists(PROBE_PATH):
        raise RuntimeError(f"{PROBE_PATH} is missing: build with `python row_wise_normalization_fp32_amd/build.py`")
    lib = ctypes.CDLL(PROBE_PATH)
    lib.rn_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.rn_probe_copy.restype = ctypes.c_int
    return lib


def stream_ceiling(read_bytes, steps, dev, geom=None, prime_ms=100.0):
    with line_marker(f"ceiling_{2 * read_bytes}"):
        return _stream_ceiling(read_bytes, steps, dev, geom, prime_ms)


def _stream_ceiling(read_bytes, steps, dev, geom=None, prime_ms=100.0):
    """Throughput of the hand-written streaming copy kernel (libstreamprobe.so) reading
    `read_bytes` and writing as many, under the same protocol as the workloads: buffer sets
    rotating over at least 1 GiB (cold L2 and memory-side cache), the kernel's own launches
    for `prime_ms`, then K launches captured in a HIP graph and replayed; the per-launch
    device time is the median of the HIP events around the replays. Checks that the copy
    is exact. This is the practical read+write ceiling at that size."""
    import torch

    geom = dict(CEILING_GEOM[read_bytes] if geom is None else geom)
    lib = probe_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid = cus * geom["per_cu"] if geom["per_cu"] > 0 else 0
    nsets = max(MIN_COLD_SETS, math.ceil(COLD_FOOTPRINT / (2 * read_bytes)))
    src = [torch.randint(0, 1 << 15, (read_bytes // 2,), dtype=torch.int16, device=dev) for _ in range(nsets)]
    dst = [torch.zeros_like(a) for a in src]
    touched = set()

    def step(i):
        touched.add(i % nsets)
        # torch's current stream at the call: inside a graph capture it is the capturing stream
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.rn_probe_copy(src[i % nsets].data_ptr(), dst[i % nsets].data_ptr(), read_bytes,
                               geom["chunks_per_lane"], geom["block_threads"], grid, geom["nontemporal"], stream)
        if st != 0:
            raise RuntimeError(f"rn_probe_copy failed with status {st}")

    torch.cuda.synchronize()
    prime_gpu(step, prime_ms)
    gt = graph_time_fn(step, steps)
    torch.cuda.synchronize()
    assert all(torch.equal(src[i], dst[i]) for i in touched), "stream probe: copy is not exact"
    del src, dst
    torch.cuda.empty_cache()
    if gt is None:
        return None
    ms = gt["event_ms"]
    gbs = 2 * read_bytes / (ms * 1e-3) / 1e9
    return {"read_bytes": read_bytes, "traffic_bytes": 2 * read_bytes, "kernel_ms": round(ms, 5),
            "GBs": round(gbs, 2), "frac": round(gbs / PEAK_HBM_GBS, 4), "replays": spread(gt), "geometry": geom}


def ceiling_sweep(steps, dev):
    """Every geometry of the copy kernel at each ceiling size (cold protocol)."""
    out = {}
    for rb in CEILING_READ_BYTES:
        rows = []
        for v in (1, 2, 4, 8):
            for b in (256, 512):
                for nt in (0, 1):
                    for per_cu in (0, 2, 4, 8):
                        g = {"chunks_per_lane": v, "block_threads": b, "per_cu": per_cu, "nontemporal": nt}
                        r = stream_ceiling(rb, steps, dev, g, prime_ms=20.0)
                        rows.append({**g, "kernel_ms": r["kernel_ms"], "GBs": r["GBs"], "frac": r["frac"],
                                     "q1_ms": r["replays"]["q1_ms"], "q3_ms": r["replays"]["q3_ms"]})
                        log(f"[bench] ceiling {2 * rb} B traffic {g}: {r['kernel_ms'] * 1e3:.2f} us, {r['frac']:.3f}")
        rows.sort(key=lambda x: x["kernel_ms"])
        out[str(2 * rb)] = rows
    return out


def copy_calibration(dev):
    """Copies of known size for scaling the HBM counters: 10 copies of 256 MiB by torch (the
    HIP runtime's copy kernel), then 10 by the streaming copy kernel of libstreamprobe.so."""
    import torch

    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    lib = probe_lib()
    for _ in range(10):
        st = lib.rn_probe_copy(src.data_ptr(), dst.data_ptr(), n, 2, 512, 0, 1, torch.cuda.current_stream().cuda_stream)
        assert st == 0, st
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 10 + 10 copies of {n} bytes")


# ---------------------------------------------------------------------------------------
# Launch-plan sweep: for each shape, the automatic plan against every alternative the library
# builds (rn_forward_tuned: waves per row, grid per row or persistent, the prefetching or the
# looping instance, the persistent grid), each timed under the lines' cold protocol. Each
# candidate runs inside a roctx range "bench:plan:<shape>:<candidate>", so that a rocprofv3
# kernel trace of the same run shows the instance and grid each one launched
# (--trace-summary).
# ---------------------------------------------------------------------------------------

PLAN_PRIME_MS = 30.0  # each candidate's own launches before its timed replays


def plan_sweep_shapes():
    import workloads

    c5, fused, fln, sm = workloads.C5, workloads.C4_FP16, workloads.FUSED_LN, workloads.SOFTMAX
    ln4k = lambda r: c5.scaled(rows=r, N=4096, name=f"ln_bf16_{r}x4096")  # noqa: E731
    return [
        (c5, "rows of 2048 chunks (8 waves x 4 chunks) with parameters, many rows: the looping instance on "
             "two workgroups per CU"),
        (c5.scaled(rows=16384, N=8192, name="ln_bf16_16384x8192"), "4-wave rows with parameters, many rows: "
                                                                   "the looping instance"),
        (ln4k(2048), "2-wave rows, few rows per resident workgroup: one workgroup per row block"),
        (ln4k(4096), "2-wave rows, 16M elements"),
        (ln4k(8192), "2-wave rows, 32M elements"),
        (ln4k(16384), "2-wave rows, 1 to 3 row blocks per resident workgroup: half as many workgroups, "
                      "prefetching"),
        (ln4k(32768), "2-wave rows, more than 3 row blocks per resident workgroup: one workgroup per row "
                      "block"),
        (fused.scaled(rows=2048, name="fused_fp16_2048x4096"), "fused add + RMSNorm (two row tensors), few rows"),
        (fused.scaled(rows=8192, name="fused_fp16_8192x4096"), "fused add + RMSNorm, more rows"),
        (fused.scaled(rows=16384, N=8192, name="fused_fp16_16384x8192"), "fused add + RMSNorm, 4-wave rows "
                                                                         "with a weight, many rows"),
        (fln.scaled(rows=8192, name="fused_ln_bf16_8192x4096"), "fused add + LayerNorm, 2-wave rows"),
        (fln.scaled(rows=16384, N=8192, name="fused_ln_bf16_16384x8192"), "fused add + LayerNorm, 4-wave rows "
                                                                          "with parameters, many rows"),
        (fln.scaled(rows=4096, N=16384, name="fused_ln_bf16_4096x16384"), "fused add + LayerNorm, 8-wave rows "
                                                                          "with parameters"),
        (sm.scaled(rows=8192, name="softmax_fp32_8192x4096"), "softmax (no parameters)"),
        (workloads.C3, "RMSNorm fp16 2048 x 4096"),
        (workloads.C1.scaled(rows=16384, name="ln_fp32_16384x1024"), "one-wave rows, four rows per "
                                                                     "workgroup"),
        (ln4k(128), "persistent threshold: 128 rows (widened to 4 waves: 128 row blocks)"),
        (ln4k(256), "persistent threshold: 256 rows (widened to 4 waves: 256 row blocks)"),
        (ln4k(384), "persistent threshold: 384 rows (widened to 4 waves: 384 row blocks)"),
        (ln4k(1024), "persistent threshold: 1024 rows (2 waves: 512 row blocks)"),
        (sm.scaled(rows=512, N=32768, name="softmax_fp32_512x32768"), "128 KiB softmax rows: one 16-wave "
                                                                       "workgroup per row against split rows"),
        (workloads.C3.scaled(rows=1024, N=65536, name="rms_fp16_1024x65536"), "128 KiB RMSNorm rows: one "
                                                                               "16-wave workgroup against split "
                                                                               "rows"),
        (c5.scaled(rows=1024, N=65536, name="ln_bf16_1024x65536"), "128 KiB LayerNorm rows: one 16-wave "
                                                                   "workgroup against split rows and the general "
                                                                   "kernel"),
        (workloads.C2.scaled(rows=1024, N=32768, name="ln_fp32_1024x32768"), "128 KiB fp32 LayerNorm rows"),
        (workloads.C4_FP16.scaled(rows=1024, N=65536, name="fused_fp16_1024x65536"), "128 KiB fused add + "
                                                                                      "RMSNorm rows"),
        (workloads.C4_BF16.scaled(rows=4096, N=65536, name="fused_bf16_4096x65536"), "128 KiB fused add + "
                                                                                     "RMSNorm rows, more rows"),
        (c5.scaled(rows=4096, N=65536, name="ln_bf16_4096x65536"), "128 KiB LayerNorm rows, more rows"),
        (sm.scaled(rows=512, N=65536, name="softmax_fp32_512x65536"), "256 KiB fp32 softmax rows: one 16-wave "
                                                                      "workgroup against split rows"),
        (workloads.C1.scaled(rows=8192, N=4095, name="ln_fp32_8192x4095"), "ragged fp32 rows: byte-addressed "
                                                                           "vectorized kernel against the element "
                                                                           "and general kernels"),
        (c5.scaled(rows=16384, N=4095, name="ln_bf16_16384x4095"), "ragged 16-bit rows: byte-addressed vectorized "
                                                                   "kernel against the pair kernel"),
        (workloads.C3.scaled(rows=16384, N=4095, name="rms_fp16_16384x4095"), "ragged RMSNorm fp16 rows"),
        (workloads.C4_BF16.scaled(rows=8192, N=4095, name="fused_bf16_8192x4095"), "ragged fused add + RMSNorm "
                                                                                  "bf16 rows"),
        (sm.scaled(rows=8192, N=4097, name="softmax_fp32_8192x4097"), "ragged fp32 softmax rows (8 waves)"),
        (c5.scaled(rows=4096, N=16383, name="ln_bf16_4096x16383"), "ragged 8-wave LayerNorm rows"),
        (workloads.C1.scaled(rows=16384, N=1023, name="ln_fp32_16384x1023"), "ragged one-wave LayerNorm rows"),
        (workloads.C3.scaled(rows=8192, N=8191, dtype="bf16", name="rms_bf16_8192x8191"), "ragged 4-wave RMSNorm "
                                                                                          "bf16 rows"),
        (workloads.C3.scaled(rows=4096, N=16383, name="rms_fp16_4096x16383"), "ragged 8-wave RMSNorm fp16 rows"),
        (workloads.C4_FP16.scaled(rows=8192, N=8191, name="fused_fp16_8192x8191"), "ragged 4-wave fused add + "
                                                                                   "RMSNorm rows"),
        (fln.scaled(rows=8192, N=8191, name="fused_ln_bf16_8192x8191"), "ragged 4-wave fused add + LayerNorm rows"),
        (sm.scaled(rows=8192, N=8191, dtype="bf16", name="softmax_bf16_8192x8191"), "ragged 4-wave bf16 softmax "
                                                                                    "rows"),
        (c5.scaled(rows=16384, N=4088, name="ln_bf16_16384x4088"), "whole-chunk rows that do not fill the row group "
                                                                   "(511 of 512 chunks): byte-addressed persistent "
                                                                   "against grid per row"),
        (workloads.C3.scaled(rows=8192, N=4092, dtype="fp32", name="rms_fp32_8192x4092"), "fp32 rows of 1023 of "
                                                                                          "1024 chunks"),
        (workloads.C3.scaled(rows=16384, N=4088, dtype="bf16", name="rms_bf16_16384x4088"), "16-bit RMSNorm rows of "
                                                                                            "511 of 512 chunks"),
        (sm.scaled(rows=16384, N=4088, dtype="bf16", name="softmax_bf16_16384x4088"), "16-bit softmax rows of 511 of "
                                                                                      "512 chunks"),
        (workloads.C4_FP16.scaled(rows=8192, N=4088, name="fused_fp16_8192x4088"), "fused add + RMSNorm rows of 511 "
                                                                                   "of 512 chunks"),
        (workloads.C1.scaled(rows=8192, N=4092, name="ln_fp32_8192x4092"), "fp32 LayerNorm rows of 1023 of 1024 "
                                                                           "chunks"),
        (c5.scaled(rows=4096, N=16376, name="ln_bf16_4096x16376"), "8-wave LayerNorm rows of 2047 of 2048 chunks"),
        (workloads.C4_FP16.scaled(rows=16384, N=4095, name="fused_fp16_16384x4095"), "ragged 2-wave fused add + "
                                                                                     "RMSNorm fp16 rows"),
        (workloads.C3.scaled(rows=4096, N=16383, dtype="fp32", name="rms_fp32_4096x16383"), "ragged 16-wave fp32 "
                                                                                            "RMSNorm rows"),
        (workloads.C1.scaled(rows=1024, N=65537, name="ln_fp32_1024x65537"), "long ragged rows: byte-addressed "
                                                                             "one-pass split rows against the "
                                                                             "element-granular two launches and "
                                                                             "the general kernel"),
        (c5.scaled(rows=1024, N=65539, name="ln_bf16_1024x65539"), "long ragged 16-bit rows (odd length)"),
        (workloads.C4_FP16.scaled(rows=1024, N=65537, name="fused_fp16_1024x65537"), "long ragged fused add + "
                                                                                     "RMSNorm rows"),
        (sm.scaled(rows=1024, N=100003, name="softmax_fp32_1024x100003"), "long ragged fp32 softmax rows"),
        # hidden sizes that are whole chunks but no power-of-two number of them (640 = 64 x 10
        # chunks, 896 = 64 x 14, ...): the row group of a power-of-two width and depth holds them
        # with idle slots
        (c5.scaled(rows=8192, N=5120, name="ln_bf16_8192x5120"), "hidden size 5120: 640 chunks = 64 x 2 x 5"),
        (workloads.C3.scaled(rows=8192, N=7168, dtype="bf16", name="rms_bf16_8192x7168"),
         "hidden size 7168: 896 chunks = 64 x 2 x 7"),
        (workloads.C4_BF16.scaled(rows=8192, N=5120, name="fused_bf16_8192x5120"),
         "fused add + RMSNorm, hidden size 5120"),
        (c5.scaled(rows=16384, N=3072, name="ln_bf16_16384x3072"), "hidden size 3072: 384 chunks = 64 x 2 x 3"),
        (workloads.C3.scaled(rows=16384, N=1536, dtype="bf16", name="rms_bf16_16384x1536"),
         "hidden size 1536: 192 chunks = 64 x 3"),
        (workloads.C1.scaled(rows=8192, N=5120, name="ln_fp32_8192x5120"), "fp32 hidden size 5120: 1280 chunks = "
                                                                           "64 x 4 x 5"),
        (fln.scaled(rows=8192, N=6144, name="fused_ln_bf16_8192x6144"), "fused add + LayerNorm, hidden size 6144: "
                                                                        "768 chunks = 64 x 4 x 3"),
        (workloads.C3.scaled(rows=4096, N=14336, dtype="bf16", name="rms_bf16_4096x14336"),
         "width 14336: 1792 chunks = 64 x 4 x 7"),
        (c5.scaled(rows=16384, N=2560, name="ln_bf16_16384x2560"), "hidden size 2560: 320 chunks = 64 x 5"),
        (c5.scaled(rows=8192, N=4608, name="ln_bf16_8192x4608"), "hidden size 4608: 576 chunks = 64 x 9"),
        (c5.scaled(rows=8192, N=6656, name="ln_bf16_8192x6656"), "hidden size 6656: 832 chunks = 64 x 13"),
        (workloads.C4_BF16.scaled(rows=8192, N=5632, name="fused_bf16_8192x5632"),
         "fused add + RMSNorm, hidden size 5632: 704 chunks = 64 x 11"),
        (workloads.C3.scaled(rows=8192, N=7680, dtype="bf16", name="rms_bf16_8192x7680"),
         "hidden size 7680: 960 chunks = 64 x 15"),
        # rows of 16 waves (64 KiB): 1024-lane workgroups, looping (no second row in registers)
        (workloads.C3.scaled(rows=4096, N=16384, dtype="fp32", name="rms_fp32_4096x16384"),
         "16-wave fp32 RMSNorm rows, persistent"),
        (workloads.C1.scaled(rows=4096, N=16384, name="ln_fp32_4096x16384"), "16-wave fp32 LayerNorm rows, "
                                                                             "persistent"),
        (sm.scaled(rows=4096, N=32768, dtype="bf16", name="softmax_bf16_4096x32768"), "16-wave bf16 softmax "
                                                                                       "rows, persistent"),
        # vocabulary-sized softmax rows: ragged (50257) and padded to whole chunks (50304)
        (sm.scaled(rows=1024, N=50257, name="softmax_fp32_1024x50257"), "vocabulary rows, not whole chunks"),
        (sm.scaled(rows=1024, N=50304, name="softmax_fp32_1024x50304"), "vocabulary rows padded to whole chunks: "
                                                                        "one 16-wave workgroup, 16 chunks per lane"),
        (workloads.C4_FP16, "persistent threshold: fused add + RMSNorm fp16 256 rows"),
        (fln.scaled(rows=384, name="fused_ln_bf16_384x4096"), "persistent threshold: fused add + LayerNorm "
                                                              "384 rows"),
        (sm.scaled(rows=256, name="softmax_fp32_256x4096"), "persistent threshold: softmax 256 rows"),
        (c5.scaled(rows=256, name="ln_bf16_256x16384"), "persistent threshold: 8-wave rows, 256 rows"),
        (c5.scaled(rows=512, name="ln_bf16_512x16384"), "persistent threshold: 8-wave rows, 512 rows"),
    ]


def _plan_ptrs(w, s0):
    ptrs = {k: s0[k].data_ptr() for k in ("x", "residual", "gamma", "beta", "weight", "y", "residual_out", "mean",
                                          "rstd") if k in s0}
    if "weight" in ptrs:
        ptrs["gamma"] = ptrs.pop("weight")
    if w.op == "softmax":
        ptrs.pop("mean", None)
        ptrs.pop("rstd", None)
    if w.op in ("rms", "fused_add_rms"):
        ptrs.pop("mean", None)
    return ptrs


def plan_candidates(rn, w, s0, cus):
    """(label, tuning, plan) for the automatic plan and each distinct built alternative."""
    import workloads

    td = workloads.TORCH_DTYPES[w.dtype]
    ptrs = _plan_ptrs(w, s0)
    st, auto = rn.plan(w.op, w.rows, w.N, td, ptrs=ptrs, eps=w.eps,
                       workspace_bytes=rn.forward_workspace_bytes(w.op, w.rows, w.N, td))
    if st != 0:
        raise RuntimeError(f"{w.name}: automatic plan failed ({rn.STATUS.get(st, st)})")
    blocks = auto["grid_blocks"]
    tries = [{"waves_per_row": W} for W in (1, 2, 4, 8, 16)]
    tries += [{"waves_per_row": W, "persistent": 0} for W in (1, 2, 4, 8, 16)]
    if auto["persistent"]:
        grids = sorted({g for g in [k * cus for k in (1, 2, 3, 4, 6, 8)] + [(blocks + 1) // 2, blocks]
                        if 0 < g <= blocks})
        tries += [{"prefetch": pf, "grid_blocks": g} for pf in (1, 0) for g in grids]
    else:
        tries.append({"persistent": 1})
    key = lambda i, t: (i["variant"], i["waves_per_row"], i["chunks_per_lane"], i["rows_per_block"],  # noqa
                        i["persistent"], i["grid_blocks"], (t or {}).get("prefetch", -1))
    out, seen = [("auto", None, auto)], {key(auto, None)}
    # the other kernel variants (forced through rn_forward_ex's variant argument), each with
    # its own automatic launch
    # (as the binding calls them: a workspace only for the split-row variants)
    ws = rn.forward_workspace_bytes(w.op, w.rows, w.N, td)
    vec = auto["variant"] in ("wave", "workgroup")
    # (byte-addressed rows are an automatic choice: forcing the wave / workgroup variant gives the
    # grid-per-row kernel of whole-chunk rows, when the rows are whole chunks)
    for v in ("element", "general", "wide", "wide_element") if vec and not auto.get("ragged") else \
            ("wave", "workgroup", "element", "general", "wide", "wide_element"):
        wsv = ws if v in ("wide", "wide_element") else 0
        st, info = rn.plan(w.op, w.rows, w.N, td, ptrs=ptrs, eps=w.eps, variant=v, workspace_bytes=wsv)
        if st != 0 or key(info, None) in seen or v == auto["variant"]:
            continue
        seen.add(key(info, None))
        out.append((f"variant {v}", {"variant": v}, info))
    if not vec:
        return out  # the tunings below apply to the vectorized variants
    for t in tries:
        st, info = rn.plan(w.op, w.rows, w.N, td, ptrs=ptrs, eps=w.eps, tuning=t)
        if st != 0 or key(info, t) in seen:
            continue
        seen.add(key(info, t))
        label = f"W{info['waves_per_row']}xV{info['chunks_per_lane']}"
        if not info["persistent"]:
            label += " grid per row"
        else:
            label += " persistent"
            if "prefetch" in t:
                label += (" prefetching" if t["prefetch"] == 1 else " looping") + f" grid {info['grid_blocks']}"
        out.append((label, t, info))
    return out


def plan_sweep(dev, steps, only=None):
    import torch

    import row_wise_normalization_fp32_amd as rn
    import workloads

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {}
    for w, why in plan_sweep_shapes():
        if only and w.name not in only:
            continue
        nbytes = workloads.algorithmic_bytes(w.op, w.rows, w.N, w.elem_bytes, with_stats=True)
        set_bytes = SET_TENSORS[w.op] * w.rows * w.N * w.elem_bytes
        nsets = max(MIN_COLD_SETS, min(64, math.ceil(COLD_FOOTPRINT / set_bytes)))
        sets = make_sets(w, nsets, dev)
        cands = plan_candidates(rn, w, sets[0], cus)
        log(f"[bench] plan sweep {w.name}: {len(cands)} plans, {nsets} buffer sets")
        rows = []
        for label, tuning, info in cands:
            step = lambda i: launch(rn, w, sets[i % nsets], tuning)  # noqa: E731
            with line_marker(f"plan:{w.name}:{label}"):
                prime_gpu(step, ms=PLAN_PRIME_MS)
                gt = graph_time_fn(step, steps)
            if gt is None:
                continue
            sp = spread({"repeats_ms": gt["repeats_ms"]})
            us = gt["event_ms"] * 1e3
            rows.append({"label": label, "tuning": tuning, "plan": info, "us": round(us, 3),
                         "q1_us": round(sp["q1_ms"] * 1e3, 3), "q3_us": round(sp["q3_ms"] * 1e3, 3),
                         "replays": sp["n"], "pct_of_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)})
        best = min(r["us"] for r in rows)
        for r in rows:
            r["vs_best"] = round(r["us"] / best, 4)
        auto = next(r for r in rows if r["label"] == "auto")
        res[w.name] = {"op": w.op, "dtype": w.dtype, "rows": w.rows, "N": w.N, "bytes": nbytes, "why": why,
                       "planner_vs_best": auto["vs_best"],
                       "planner_rank": 1 + sum(r["us"] < auto["us"] for r in rows), "candidates": rows}
        log(f"[bench] plan sweep {w.name}: planner {auto['us']:.2f} us, best {best:.2f} us "
            f"({auto['vs_best']:.3f}x)")
        del sets
        torch.cuda.empty_cache()
    return {"cus": cus, "steps": steps, "replay_ms": MIN_REPLAY_MS, "prime_ms": PLAN_PRIME_MS, "shapes": res}


def trace_by_range(trace_dir):
    """Kernel dispatches of a rocprofv3 --kernel-trace --marker-trace run, grouped by the
    roctx range ("bench:...") whose host-time span contains each dispatch's start: per range,
    per kernel, (dispatches, median duration in us of the last 100, workgroups). torch's own
    helper kernels are left out."""
    import bisect
    import csv
    import statistics

    marks = [r for r in csv.DictReader(open(os.path.join(trace_dir, "trace_marker_api_trace.csv")))
             if r["Function"].startswith("bench:")]
    marks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Function"][6:]) for r in marks)
    starts = [m[0] for m in marks]
    by = {m[2]: {} for m in marks}
    kt = os.path.join(trace_dir, "trace_kernel_trace.csv")
    if not os.path.exists(kt) and os.path.exists(kt + ".gz"):  # kept compressed
        import gzip

        kfile = gzip.open(kt + ".gz", "rt")
    else:
        kfile = open(kt)
    for r in csv.DictReader(kfile):
        t = int(r["Start_Timestamp"])
        i = bisect.bisect_right(starts, t) - 1
        if i < 0 or t > marks[i][1]:
            continue
        # the template name: no return type, no argument list
        name = re.sub(r"\(.*$", "", r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", ""))
        if name.startswith("at::") or name.startswith("__amd"):
            continue
        wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        wg *= int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(1, int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        by[marks[i][2]].setdefault((name, wg), []).append((t, int(r["End_Timestamp"]) - t))
    out = {}
    for rng, ks in by.items():
        rowsk = []
        for (name, wg), v in ks.items():
            v.sort()
            rowsk.append((v[0][0], name, len(v), statistics.median(d for _, d in v[-100:]) / 1e3, wg))
        out[rng] = [(n, c, us, wg) for _, n, c, us, wg in sorted(rowsk)]
    return out


def trace_summary(trace_dir):
    """Markdown table of trace_by_range: the kernels launched at least 20 times in a range (a
    range's other kernels prepare its inputs), and for a bench line the sum per step with the
    line's algorithmic bytes per second."""
    import workloads

    wl = bench_workloads()
    lines = ["| range | kernel (template arguments) | workgroups | dispatches | median µs (last 100) | "
             "µs per step | GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|---|---|"]
    for rng, ks in trace_by_range(trace_dir).items():
        ks = [k for k in ks if k[1] >= 20]
        if not ks:
            continue
        line = rng.partition(":")[0]
        b = None
        if line.startswith("ceiling_"):
            b = int(line.split("_")[1])
        elif line in wl and not rng.startswith("plan:"):
            w = wl[line]
            b = workloads.algorithmic_bytes(w.op, w.rows, w.N, w.elem_bytes, with_stats=True)
        tot = sum(k[2] for k in ks)
        for i, (name, c, us, wg) in enumerate(ks):
            tail = " | | |"
            if i == len(ks) - 1:
                gbs = b / (tot * 1e-6) / 1e9 if b else None
                tail = (f" {tot:.2f} | " + (f"{gbs:.0f} | {100 * gbs / PEAK_HBM_GBS:.1f} |" if gbs else " | |"))
            lines.append(f"| {rng} | `{name}` | {wg} | {c} | {us:.2f} |" + tail)
    return "\n".join(lines)


def _csv_rows(path):
    """Rows of a rocprofv3 CSV, read from `path` or from `path`.gz."""
    import csv
    import gzip

    f = gzip.open(path + ".gz", "rt") if not os.path.exists(path) and os.path.exists(path + ".gz") else open(path)
    with f:
        return list(csv.DictReader(f))


def _counter_medians(run_dir, prefix):
    """Median counter value per (kernel template name, workgroups) of a --pmc run."""
    import statistics

    by = {}
    for r in _csv_rows(os.path.join(run_dir, f"{prefix}_counter_collection.csv")):
        name = re.sub(r"\(.*$", "", r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", ""))
        wg = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
        by.setdefault((name, wg), []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in by.items()}


def bench_workloads():
    """Every workload a default run of this script times, by line name (as line_marker names
    its roctx range without the cache suffix)."""
    import workloads

    ws = [workloads.C5, workloads.FUSED_8192] + [x for _, x, _ in _more()] + list(workloads.CONFIGS)
    ws += [workloads.C4_FP16.scaled(rows=r, name=f"fused_fp16_{r}x4096") for r in (2048, 8192, 32768)]
    ws += [workloads.C4_BF16.scaled(rows=r, name=f"fused_bf16_{r}x4096") for r in (2048, 8192, 32768)]
    ws += [workloads.C5.scaled(rows=r, N=4096, name=f"ln_bf16_{r}x4096") for r in (2048, 4096, 8192)]
    ws += [workloads.C5.scaled(name="ln_bf16_4096x16384_hot")]
    return {w.name: w for w in ws}


def traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, trace_dir):
    """HBM traffic per call of each bench line from two --pmc runs of this script (FETCH_SIZE,
    WRITE_SIZE, KiB per dispatch), scaled by what the same counters read for the streaming
    copy kernel of --copy-calibration (256 MiB read and written per dispatch), with each
    kernel attributed to its line through a --kernel-trace --marker-trace run. The text is the
    record counter_traffic() reads."""
    import statistics
    import workloads

    cal = {}
    for c, d in (("FETCH_SIZE", cal_fetch_dir), ("WRITE_SIZE", cal_write_dir)):
        v = [float(r["Counter_Value"]) for r in _csv_rows(os.path.join(d, "cal_counter_collection.csv"))
             if "stream_copy" in r["Kernel_Name"]]
        cal[c] = (256 * 1024) / statistics.median(v)
    cnt = {"FETCH_SIZE": _counter_medians(fetch_dir, "pmc"), "WRITE_SIZE": _counter_medians(write_dir, "pmc")}
    by = trace_by_range(trace_dir)
    wl = bench_workloads()
    out = [f"kernel_source_sha256_16: {kernel_source_hash()}",
           "# (sha256 of rownorm_kernels.hpp + rownorm_backward.hpp + rownorm_capi.cpp with comments",
           "# and whitespace removed; bench.py reports traffic only while it matches)",
           f"# fetch scale {cal['FETCH_SIZE']:.5f}, write scale {cal['WRITE_SIZE']:.5f} (streaming copy: "
           f"FETCH_SIZE {256 * 1024 / cal['FETCH_SIZE']:.1f} KiB, WRITE_SIZE {256 * 1024 / cal['WRITE_SIZE']:.1f} KiB "
           "per 262144 KiB read and written)", ""]
    seen = set()
    for rng, ks in by.items():
        if rng.startswith("plan:"):
            continue
        line, _, cache = rng.partition(":")
        key = "ln_bf16_4096x16384" if line in ("C5_ln_bf16_4096x16384", "ln_bf16_4096x16384_hot") else line
        if cache == "hot" or key in seen:
            continue
        seen.add(key)
        if line.startswith("ceiling_"):
            b = int(line.split("_")[1])
        elif line in wl:
            w = wl[line]
            b = workloads.algorithmic_bytes(w.op, w.rows, w.N, w.elem_bytes, with_stats=True)
        else:
            continue
        t, desc = 0.0, []
        for name, n, _, wg in ks:
            if n < 20:
                continue  # launched only to prepare a line's inputs
            f, w_ = cnt["FETCH_SIZE"].get((name, wg)), cnt["WRITE_SIZE"].get((name, wg))
            if f is None or w_ is None:
                desc.append(f"#   {name} ({wg} workgroups): no counter record")
                t = None
                break
            t += (f * cal["FETCH_SIZE"] + w_ * cal["WRITE_SIZE"]) * 1024
            desc.append(f"#   {name} ({wg} workgroups): FETCH_SIZE {f:.1f} KiB, WRITE_SIZE {w_:.1f} KiB")
        out.append(f"# {key}" + (" (streaming copy, bytes read + written)" if line.startswith("ceiling_") else ""))
        out.extend(desc)
        if t is not None:
            out.append(f"#   algorithmic bytes {b}; measured/algorithmic = {t / b:.4f}")
            out.append(f"{key} traffic_bytes_per_launch: {t:.0f}")
        out.append("")
    return "\n".join(out)


def plan_sweep_report(sweep, trace_dir=None, top=0):
    """Markdown tables of a --plan-sweep result (and, with its trace, the kernel instance and
    grid each candidate launched with their traced durations); top > 0: per shape only the
    `top` fastest plans, the planner's and the slowest."""
    tr = trace_by_range(trace_dir) if trace_dir else {}
    out = []
    ratios = []
    for name, r in sweep["shapes"].items():
        out.append(f"### {name} ({r['op']}, {r['dtype']}, {r['rows']} x {r['N']}): {r['why']}")
        out.append("")
        out.append(f"Planner: {r['planner_vs_best']:.3f}x the fastest plan (rank {r['planner_rank']} of "
                   f"{len(r['candidates'])}).")
        out.append("")
        hdr = "| plan | µs (events, median) | % of 8 TB/s | vs fastest |"
        sep = "|---|---|---|---|"
        if tr:
            hdr += " kernel instance (trace) | workgroups | µs (trace) |"
            sep += "---|---|---|"
        out += [hdr, sep]
        ratios.append(r["planner_vs_best"])
        cands = sorted(r["candidates"], key=lambda c: c["us"])
        if top > 0:
            cands = [c for i, c in enumerate(cands) if i < top or i == len(cands) - 1 or c["label"] == "auto"]
        for c in cands:
            lab = "**planner** (" + _plan_label(c["plan"]) + ")" if c["label"] == "auto" else c["label"]
            line = f"| {lab} | {c['us']:.2f} | {c['pct_of_peak']:.1f} | {c['vs_best']:.3f} |"
            if tr:
                ks = [k for k in tr.get(f"plan:{name}:{c['label']}", []) if k[1] >= 20]
                line += (" " + " + ".join(f"`{k[0]}`" for k in ks) + " | " + " + ".join(str(k[3]) for k in ks) +
                         " | " + f"{sum(k[2] for k in ks):.2f} |")
            out.append(line)
        out.append("")
    gm = math.exp(sum(math.log(x) for x in ratios) / len(ratios)) if ratios else float("nan")
    head = [f"Planner against the fastest built plan over {len(ratios)} shapes: geometric mean "
            f"{gm:.3f}x, worst {max(ratios):.3f}x.", ""]
    return "\n".join(head + out)


def _plan_label(info):
    if info["variant"] not in ("wave", "workgroup"):
        return f"{info['variant']} variant"
    s = f"W{info['waves_per_row']}xV{info['chunks_per_lane']}"
    return s + (" persistent, grid rule" if info["persistent"] else " grid per row")


def _more():
    import workloads

    return [
        ("fused_add_layer_norm", workloads.FUSED_LN_8192,
         "fused residual-add + LayerNorm, bf16 I/O, 8192 x 4096, eps 1e-5, y + residual_out + mean + rstd"),
        ("softmax", workloads.SOFTMAX_8192.scaled(name="softmax_fp32_8192x4096"),
         "row-wise softmax, fp32 I/O, 8192 x 4096"),
        ("ln_backward", workloads.LN_BWD,
         "LayerNorm backward, bf16 I/O, 4096 x 16384: dx, dgamma, dbeta from fp32 mean / rstd"),
        ("rms_norm_backward", workloads.RMS_BWD.scaled(rows=8192, name="rms_bwd_fp16_8192x4096"),
         "RMSNorm backward, fp16 I/O, 8192 x 4096: dx, dweight from fp32 rstd"),
        ("layer_norm_ragged", workloads.LN_RAGGED,
         "LayerNorm, bf16 I/O, 16384 x 4095 (rows not whole 16-byte chunks: the vectorized kernel with "
         "byte-addressed rows, 16-byte accesses at 2-byte alignment), y + mean + rstd"),
        ("layer_norm_split_rows", workloads.LN_SPLIT,
         "LayerNorm, fp32 I/O, 1024 x 65536 (rows beyond a workgroup's registers: one-pass split rows, the "
         "segments of a row exchanging their statistics through the workspace, x read once)"),
        ("softmax_vocab", workloads.SOFTMAX_VOCAB,
         "row-wise softmax, fp32 I/O, 1024 x 50257 (vocabulary-sized rows, not whole chunks: byte-addressed rows, "
         "one 16-wave workgroup per row)"),
        ("ln_backward_split_rows", workloads.LN_BWD.scaled(rows=1024, N=65536, name="ln_bwd_bf16_1024x65536"),
         "LayerNorm backward, bf16 I/O, 1024 x 65536 (rows beyond one workgroup: one launch in which the "
         "segments of a row exchange their sums through the workspace, x and dy read once; then column sums)"),
    ]


def main():
    global MORE, MIN_REPLAY_MS, PRIME_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cache", choices=["cold", "hot"], default="cold")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-more", action="store_true", help="skip the fused LayerNorm, softmax and backward lines")
    ap.add_argument("--no-sweep", action="store_true", help="skip the scale-up sweep and the hot-cache line")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration throughput block")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="time every geometry of the streaming copy kernel at the ceiling sizes, print JSON, exit")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-copy ceiling lines")
    ap.add_argument("--plan-sweep", action="store_true",
                    help="time the automatic launch plan of several shapes against every built alternative, "
                         "print JSON, exit")
    ap.add_argument("--shapes", metavar="NAMES", help="--plan-sweep: only these shapes (comma-separated names)")
    ap.add_argument("--plan-sweep-report", metavar="JSON",
                    help="markdown tables of a --plan-sweep result (with --trace DIR: and of its kernel trace)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="markdown table of a rocprofv3 --kernel-trace --marker-trace run of this script")
    ap.add_argument("--trace", metavar="DIR", help="the kernel trace of the --plan-sweep run (for the report)")
    ap.add_argument("--traffic-summary", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR",
                                                            "TRACE_DIR"),
                    help="HBM traffic per bench line from --pmc FETCH_SIZE / WRITE_SIZE runs of this script, the "
                         "--copy-calibration runs and a --kernel-trace --marker-trace run")
    ap.add_argument("--top", type=int, default=0, help="report: per shape the fastest N plans, the planner's and "
                                                       "the slowest")
    ap.add_argument("--prime-ms", type=float, default=PRIME_MS,
                    help="the workload's own launches before each line (shorter for counter runs)")
    ap.add_argument("--replay-ms", type=float, default=MIN_REPLAY_MS,
                    help="device time the timed graph replays of a line add up to (at least 5 replays)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "rows are independent, so more GPUs would each run the same kernel on their own rows.",
              file=sys.stderr)
        sys.exit(2)

    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary))
        return
    if args.plan_sweep_report:
        sweep = json.loads(open(args.plan_sweep_report).read().strip().splitlines()[-1])["plan_sweep"]
        print(plan_sweep_report(sweep, args.trace, args.top))
        return

    import torch

    import workloads

    MORE = _more()
    MIN_REPLAY_MS = args.replay_ms
    PRIME_MS = args.prime_ms
    dev = "cuda:0"
    if args.copy_calibration:
        copy_calibration(dev)
        return
    if args.ceiling_sweep:
        print(json.dumps({"ceiling_sweep": ceiling_sweep(args.steps, dev)}), flush=True)
        return
    if args.plan_sweep:
        only = set(args.shapes.split(",")) if args.shapes else None
        print(json.dumps({"plan_sweep": plan_sweep(dev, args.steps, only)}), flush=True)
        return

    w = workloads.C5
    log(f"[bench] timing {w.name} ({args.cache} cache) ...")
    r = measure(w, args.steps, args.warmup, args.cache, dev)
    value = r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
    kms, timing = kernel_time(r)
    achieved = r["bytes"] / (kms * 1e-3) / 1e9
    traffic = counter_traffic("ln_bf16_4096x16384")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "LayerNorm forward, bf16 I/O, 4096 x 16384, eps 1e-5, y + fp32 mean/rstd",
            "op": "ln_forward", "io_dtype": "bf16", "rows": w.rows, "N": w.N, "cache": args.cache,
            "buffer_sets": r["nsets"], "variant": r["plan"]["variant"], "persistent": r["plan"]["persistent"],
            "inputs": "x = m_r + s_r*z, m_r~U(-10,10), s_r~U(0.5,4); gamma~U(0.5,1.5); beta~N(0,0.1^2); seed 1005",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "rows_per_s": round(w.rows / (r["ms_per_step"] * 1e-3), 1),
        "timing": TIMING[r["timing"]],
        "eager": eager_fields(r),
        "replays": spread(r),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": kernel_name(w, r["plan"]),
            "kernel_avg_ms": round(kms, 5), "kernel_timing": timing,
            "stream_ms_per_launch": round(r["kernel_ms"], 5),
            "bytes_per_launch": r["bytes"],
        },
        "cpu_baseline": None,
    }
    if not args.no_fused:
        f = workloads.FUSED_8192
        log(f"[bench] timing {f.name} ({args.cache} cache) ...")
        rf = measure(f, args.steps, args.warmup, args.cache, dev)
        fv = rf["bytes"] / (rf["ms_per_step"] * 1e-3) / 1e9
        fkms, _ = kernel_time(rf)
        fa = rf["bytes"] / (fkms * 1e-3) / 1e9
        out["fused_add_rms_norm"] = {
            "workload": "fused residual-add + RMSNorm, fp16 I/O, 8192 x 4096, eps 1e-6, y + residual_out + rstd",
            "value": round(fv, 2), "unit": "GB/s", "pct_of_peak": round(100.0 * fv / PEAK_HBM_GBS, 2),
            "rows_per_s": round(f.rows / (rf["ms_per_step"] * 1e-3), 1), "ms_per_step": round(rf["ms_per_step"], 5),
            "kernel_avg_ms": round(fkms, 5), "stream_ms_per_launch": round(rf["kernel_ms"], 5),
            "achieved_kernel_GBs": round(fa, 2),
            "frac_kernel": round(fa / PEAK_HBM_GBS, 4), "bytes_per_launch": rf["bytes"],
            "kernel": kernel_name(f, rf["plan"]), "traffic": counter_traffic("fused_fp16_8192x4096"),
            "timing": rf["timing"], "eager": eager_fields(rf), "replays": spread(rf),
        }
    if not args.no_more:
        more = {}
        extra_steps = min(args.steps, 100)
        for key, x, what in MORE:
            log(f"[bench] timing {x.name} ({args.cache} cache) ...")
            rx = measure(x, extra_steps, min(args.warmup, 10), args.cache, dev)
            xv = rx["bytes"] / (rx["ms_per_step"] * 1e-3) / 1e9
            xkms, _ = kernel_time(rx)
            xa = rx["bytes"] / (xkms * 1e-3) / 1e9
            more[key] = {
                "workload": what, "value": round(xv, 2), "unit": "GB/s",
                "pct_of_peak": round(100.0 * xv / PEAK_HBM_GBS, 2), "ms_per_step": round(rx["ms_per_step"], 5),
                "steps": extra_steps, "kernel_avg_ms": round(xkms, 5),
                "stream_ms_per_launch": round(rx["kernel_ms"], 5),
                "achieved_kernel_GBs": round(xa, 2), "frac_kernel": round(xa / PEAK_HBM_GBS, 4),
                "bytes_per_launch": rx["bytes"], "rows_per_s": round(x.rows / (rx["ms_per_step"] * 1e-3), 1),
                "kernel": kernel_name(x, rx["plan"]),
                # HBM bytes per call from the counter record (backward: row + column kernels)
                "traffic": counter_traffic(x.name),
                "timing": rx["timing"], "eager": eager_fields(rx), "replays": spread(rx),
            }
        out["more"] = more
    if not args.no_configs:
        # Every configuration the target lists (C1-C5, C4 in fp16 and bf16): rows/s and
        # GB/s with % of peak, cold (rotating buffers) and hot (one buffer set), from HIP
        # events per launch and from a replayed HIP graph (device time without host gaps),
        # next to the oracle on the host cores (a baseline, not the target).
        confs = {}
        for c in workloads.CONFIGS:
            entry = {"rows": c.rows, "N": c.N, "dtype": c.dtype, "op": c.op}
            for cache in ("cold", "hot"):
                rc = measure(c, min(args.steps, 100), min(args.warmup, 10), cache, dev, graph=True)
                gm = rc["graph_ms"]
                entry[cache] = {
                    "kernel_avg_ms": round(rc["kernel_ms"], 5),
                    "graph_ms": None if gm is None else round(gm, 5),
                    "GBs_graph": None if gm is None else round(rc["bytes"] / (gm * 1e-3) / 1e9, 2),
                    "pct_of_peak_graph": None if gm is None else round(100 * rc["bytes"] / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                    "rows_per_s_graph": None if gm is None else round(c.rows / (gm * 1e-3), 1),
                    "GBs_events": round(rc["bytes"] / (rc["kernel_ms"] * 1e-3) / 1e9, 2),
                }
            entry["bytes_per_call"] = rc["bytes"]
            confs[c.name] = entry
        out["configs"] = confs
    if not args.no_sweep:
        # The scale-up sweep of the 8M-element target clause (fused add + RMSNorm at N = 4096,
        # fp16 and bf16, 2048 / 8192 / 32768 rows; LayerNorm bf16 at N = 4096, 2048 / 4096 /
        # 8192 rows), cold cache, and the headline workload hot (one buffer set, re-launched
        # back to back).
        sweep = {}
        cases = [(workloads.C4_FP16.scaled(rows=r, name=f"fused_fp16_{r}x4096"), "cold") for r in (2048, 8192, 32768)]
        cases += [(workloads.C4_BF16.scaled(rows=r, name=f"fused_bf16_{r}x4096"), "cold") for r in (2048, 8192, 32768)]
        cases += [(workloads.C5.scaled(rows=r, N=4096, name=f"ln_bf16_{r}x4096"), "cold") for r in (2048, 4096, 8192)]
        cases += [(workloads.C5.scaled(name="ln_bf16_4096x16384_hot"), "hot")]
        for x, cache in cases:
            log(f"[bench] sweep {x.name} ({cache}) ...")
            rx = measure(x, min(args.steps, 100), min(args.warmup, 10), cache, dev, graph=True)
            xa = rx["bytes"] / (rx["kernel_ms"] * 1e-3) / 1e9
            xv = rx["bytes"] / (rx["eager_ms_per_step"] * 1e-3) / 1e9
            gm = rx["graph_ms"]
            sweep[x.name] = {"elements": x.rows * x.N, "cache": cache, "bytes": rx["bytes"],
                             # eager launches: HIP events around the K timed launches
                             "stream_ms_per_launch": round(rx["kernel_ms"], 5),
                             "frac_stream": round(xa / PEAK_HBM_GBS, 4),
                             # wall clock over the eager launches
                             "value": round(xv, 2), "pct_of_peak": round(100.0 * xv / PEAK_HBM_GBS, 2),
                             # device time per launch from a replayed HIP graph (no host gaps)
                             "graph_ms": None if gm is None else round(gm, 5),
                             "frac_graph": None if gm is None else round(rx["bytes"] / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        out["scale_up_sweep"] = sweep
    if not args.no_ceiling:
        # The hand-written streaming copy kernel at the traffic of LayerNorm bf16 at 8M
        # elements, fused add + RMSNorm at 8M elements and the 4096 x 16384 LayerNorm, under
        # the same cold protocol: the practical read+write ceiling at each size.
        ceil = {}
        for rb in CEILING_READ_BYTES:
            log(f"[bench] ceiling: streaming copy of {rb} bytes ...")
            c = stream_ceiling(rb, min(args.steps, 100), dev)
            if c is not None:
                ceil[str(2 * rb)] = c
        out["ceiling"] = {"what": "hand-written streaming copy kernel (libstreamprobe.so), same protocol as the "
                                  "lines; key = bytes moved per launch (read + write)", "sizes": ceil}
        by_traffic = {int(k): v for k, v in ceil.items()}

        def vs_ceiling(nbytes, ms):
            t = min(by_traffic, key=lambda k: abs(k - nbytes), default=None)
            if t is None or abs(t - nbytes) > 0.02 * nbytes or not ms:
                return None
            return round((nbytes / ms) / (t / by_traffic[t]["kernel_ms"]), 4)

        out["roofline"]["frac_of_ceiling"] = vs_ceiling(r["bytes"], kms)
        for x in out.get("scale_up_sweep", {}).values():
            bx = x.get("bytes")
            if bx and x.get("graph_ms"):
                x["graph_frac_of_ceiling"] = vs_ceiling(bx, x["graph_ms"])
        for x in out.get("configs", {}).values():
            if x.get("cold", {}).get("graph_ms"):
                x["cold"]["graph_frac_of_ceiling"] = vs_ceiling(x["bytes_per_call"], x["cold"]["graph_ms"])
    # The CPU baseline last: the oracle on the host cores keeps the GPU idle for seconds,
    # so it runs after every GPU line instead of before the headline.
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(workloads.C5, args.cpu_seconds, single_thread=True)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")
        for c in workloads.CONFIGS if "configs" in out else ():
            cb = cpu_baseline(c, min(args.cpu_seconds, 1.0))
            out["configs"][c.name]["cpu_oracle"] = {"rows_per_s": cb["rows_per_s"], "GBs": cb["value"],
                                                    "cores": cb["cores"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
