"""rn_forward_noalloc (include/rownorm.h): the forward entry point that allocates nothing and
takes the split-row workspace from the library's static per-GPU array. Called through the C
ABI with device pointers, checked bit for bit against rn_forward_ex with a caller workspace
(the same kernels) and against the fp64 oracle, on two calls in a row, the second smaller."""

import ctypes
import os

import pytest
import torch

import oracle
import row_wise_normalization_fp32_amd as rn
import workloads
from _compare import check_bits_equal, check_mean, check_rstd, check_y

DEV = "cuda:0"
THREADS = min(16, os.cpu_count() or 1)
LIB = rn._lib
OPS = {"ln": 0, "rms": 1, "fused_add_rms": 2, "fused_add_ln": 3}
DT = {"fp32": 0, "fp16": 1, "bf16": 2}
SCRATCH = 9  # RN_ERR_SCRATCH


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(fn, w, g, outs, extra=()):
    rows, N = w.rows, w.N
    return fn(OPS[w.op], _p(g["x"]), _p(g.get("residual")), _p(g.get("gamma", g.get("weight"))), _p(g.get("beta")),
              _p(outs["y"]), _p(outs.get("residual_out")), _p(outs.get("mean")), _p(outs["rstd"]), rows, N,
              ctypes.c_float(w.eps), DT[w.dtype], None, *extra, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _outs(w, g):
    o = {"y": torch.full_like(g["x"], float("nan")), "rstd": torch.full((w.rows,), float("nan"), device=DEV)}
    if w.op in ("ln", "fused_add_ln"):
        o["mean"] = torch.full((w.rows,), float("nan"), device=DEV)
    if w.op in ("fused_add_rms", "fused_add_ln"):
        o["residual_out"] = torch.full_like(g["x"], float("nan"))
    return o


def _equal(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                       b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))


def _oracle(w, inp):
    if w.op == "ln":
        return oracle.layer_norm(inp["x"], inp.get("gamma"), inp.get("beta"), w.eps, threads=THREADS)
    if w.op == "rms":
        return oracle.rms_norm(inp["x"], inp.get("weight"), w.eps, threads=THREADS)
    if w.op == "fused_add_rms":
        return oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp.get("weight"), w.eps, threads=THREADS)
    return oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp.get("gamma"), inp.get("beta"), w.eps,
                                       threads=THREADS)


def _case(w):
    """rn_forward_noalloc against rn_forward_ex with a workspace (bits) and the oracle."""
    inp = workloads.make_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    need = int(LIB.rn_forward_workspace_bytes(OPS[w.op], w.rows, w.N, DT[w.dtype]))
    a, b = _outs(w, g), _outs(w, g)
    st = _call(LIB.rn_forward_noalloc, w, g, a)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    st2 = _call(LIB.rn_forward_ex, w, g, b, (0, ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need)))
    torch.cuda.synchronize()
    assert st == 0 and st2 == 0, (rn.STATUS.get(st), rn.STATUS.get(st2))
    for k in a:
        assert _equal(a[k], b[k]), k
    ref = _oracle(w, inp)
    check_y(a["y"], ref["y"], "y", op=w.op)
    check_rstd(a["rstd"], ref["rstd"])
    if "mean" in a:
        check_mean(a["mean"], ref["mean"], ref["rstd"], w.eps)
    if "residual_out" in a:
        check_bits_equal(a["residual_out"], ref["residual_out"], "residual_out")
    return need


@pytest.mark.gpu
def test_no_alloc_matches_workspace_entry_point_twice_second_smaller():
    # split rows of whole 16-byte chunks (32 KiB segments), then a smaller call whose rows are
    # not whole chunks (8192-element segments): both take their workspace from the scratch
    first = workloads.C2.scaled(rows=96, N=65536, seed=1501)                # LN fp32, 8 segments
    second = workloads.C5.scaled(rows=24, N=40001, seed=1502)               # LN bf16, 5 element segments
    assert _case(first) > _case(second) > 0
    # the fused ops and RMSNorm over the same scratch, and a shape that needs none
    _case(workloads.FUSED_LN.scaled(rows=40, N=50000, seed=1503))
    _case(workloads.C4_FP16.scaled(rows=32, N=98304, seed=1504))
    _case(workloads.C3.scaled(rows=16, N=70000, seed=1505))
    assert _case(workloads.C3.scaled(rows=64, N=4096, seed=1506)) == 0


def test_no_alloc_rejects_shapes_beyond_the_scratch_before_any_launch():
    # 2^20 rows of 2^17 elements need 16 records per row (256 MiB of workspace): rejected on
    # the host, before any pointer is used or anything is enqueued
    assert LIB.rn_forward_noalloc(0, ctypes.c_void_p(1 << 20), None, None, None, ctypes.c_void_p(1 << 40), None, None,
                                  None, 1 << 20, 1 << 17, ctypes.c_float(1e-5), 0, None, None) == SCRATCH
    # exactly at the limit the size check passes (the argument checks of rn_forward_ex follow:
    # a NULL x is reported as such, still before any launch)
    rows = ((16 << 20) - 256) // (8 * 32)  # one-pass layout: 256-byte header, 32 bytes per segment record
    assert int(LIB.rn_forward_workspace_bytes(0, rows, 65536, 0)) == 16 << 20
    assert LIB.rn_forward_noalloc(0, None, None, None, None, ctypes.c_void_p(1 << 40), None, None, None, rows, 65536,
                                  ctypes.c_float(1e-5), 0, None, None) == 1
    assert rn.STATUS[SCRATCH] == "RN_ERR_SCRATCH"
    assert LIB.rn_status_string(SCRATCH) == b"RN_ERR_SCRATCH"
