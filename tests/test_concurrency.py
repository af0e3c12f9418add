"""Several host threads calling the library at once, each on its own HIP stream (the entry
points keep no state besides per-device occupancy caches, which are guarded): every result
must equal, bit for bit, the same call made alone."""

import threading

import pytest
import torch

import row_wise_normalization_fp32_amd as rn
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _calls():
    ln = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.C5.scaled(rows=2048)).items()}
    fr = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.FUSED_8192.scaled(rows=4096)).items()}
    rg = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.LN_RAGGED.scaled(rows=4096)).items()}
    wd = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.LN_SPLIT.scaled(rows=64)).items()}
    bw = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.LN_BWD.scaled(rows=512, N=4096)).items()}
    _, m, r = rn.ln_forward(bw["x"], None, None, 1e-5, return_stats=True)
    sb = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.LN_BWD.scaled(rows=256, N=65536)).items()}
    _, m2, r2 = rn.ln_forward(sb["x"], None, None, 1e-5, return_stats=True)
    torch.cuda.synchronize()
    return [
        lambda: [rn.ln_forward(ln["x"], ln["gamma"], ln["beta"], 1e-5)],  # persistent vectorized
        lambda: list(rn.fused_add_rms_norm(fr["x"], fr["residual"], fr["weight"], 1e-6)),
        lambda: [rn.ln_forward(rg["x"], rg["gamma"], rg["beta"], 1e-5)],  # persistent pairs
        lambda: [rn.ln_forward(wd["x"], wd["gamma"], wd["beta"], 1e-5)],  # split rows + workspace
        lambda: list(rn.ln_backward(bw["dy"], bw["x"], m, r, bw["gamma"])),  # row + column kernels
        # split rows in one pass: tickets and records in each call's own workspace, calls
        # on other streams competing for the compute units meanwhile
        lambda: list(rn.ln_backward(sb["dy"], sb["x"], m2, r2, sb["gamma"])),
    ]


def _bits(ts):
    return [t.contiguous().view(torch.uint8).clone() for t in ts]


def test_threads_on_their_own_streams():
    calls = _calls()
    alone = []
    for c in calls:
        alone.append(_bits(c()))
        torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(6):
                    c = calls[(k + it) % len(calls)]
                    out = _bits(c())
                    s.synchronize()
                    want = alone[(k + it) % len(calls)]
                    for a, b in zip(out, want):
                        if not torch.equal(a, b):
                            errors.append((k, it))
        except Exception as e:  # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    assert not errors, errors
