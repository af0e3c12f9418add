"""The entry points under HIP graph capture (torch.cuda.graph): a captured call sequence is
replayed several times, with eager work (clearing the outputs) and synchronizations between
the replays, and every replay must reproduce the eager results bit for bit. The library
records only kernel launches (no memset or copy nodes), so replays recompute everything.
"""

import pytest
import torch

import row_wise_normalization_fp32_amd as rn
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).clone()


def test_graph_replays_match_eager():
    ln = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.C5.scaled(rows=4096)).items()}
    fr = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.FUSED_8192).items()}
    fl = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.FUSED_LN.scaled(rows=512)).items()}
    sm = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.SOFTMAX).items()}
    wide = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.C5.scaled(rows=4, N=131072)).items()}
    wel = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.C2.scaled(rows=4, N=50257)).items()}
    bw = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.LN_BWD.scaled(rows=256, N=4096)).items()}
    bl = {k: v.to(DEV) for k, v in workloads.make_inputs(workloads.RMS_BWD.scaled(rows=8, N=40000)).items()}
    be = {k: v.to(DEV) for k, v in workloads.make_inputs(
        workloads.LN_BWD.scaled(rows=6, N=40001, dtype="bf16")).items()}

    def run():
        y1, m1, r1 = rn.ln_forward(ln["x"], ln["gamma"], ln["beta"], 1e-5, return_stats=True)
        y2, ro2 = rn.fused_add_rms_norm(fr["x"], fr["residual"], fr["weight"], 1e-6)
        y3, ro3 = rn.fused_add_layer_norm(fl["x"], fl["residual"], fl["gamma"], fl["beta"], 1e-5)
        y4 = rn.softmax_forward(sm["x"])
        # split rows in one pass: clear and one-pass launches (the clear kernel resets the
        # ticket counter and the records on every replay)
        y5 = rn.ln_forward(wide["x"], wide["gamma"], wide["beta"], 1e-5)
        y7 = rn.ln_forward(wel["x"], wel["gamma"], wel["beta"], 1e-5)  # split rows at element granularity
        _, m6, r6 = rn.ln_forward(bw["x"], None, None, 1e-5, return_stats=True)
        dx, dg, db = rn.ln_backward(bw["dy"], bw["x"], m6, r6, bw["gamma"])  # row + column kernels
        _, r8 = rn.rms_norm(bl["x"], None, 1e-6, return_rstd=True)
        # split rows in one pass (clear, one-pass and column launches; the clear kernel resets
        # the ticket counter on every replay)
        dx8, dw8 = rn.rms_norm_backward(bl["dy"], bl["x"], r8, bl["weight"])
        _, m9, r9 = rn.ln_forward(be["x"], None, None, 1e-5, return_stats=True)
        # 16-bit split rows that are not whole 16-byte groups: statistics, dx, column launches
        dx9, dg9, db9 = rn.ln_backward(be["dy"], be["x"], m9, r9, be["gamma"])
        return [y1, m1, r1, y2, ro2, y3, ro3, y4, y5, y7, dx, dg, db, dx8, dw8, dx9, dg9, db9]

    eager = [_bits(t) for t in run()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the side stream (occupancy queries, allocator)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for rep in range(3):
        for o in outs:
            o.view(torch.uint8).fill_(0xFF)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(_bits(o), e), f"replay {rep}: output {i} differs from the eager result"
