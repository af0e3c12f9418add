"""GPU parity through the plain C entry points of include/rownorm.h (ln_forward, rms_norm,
fused_add_rms_norm, and fused_add_layer_norm / softmax_forward), called directly through
ctypes with device pointers from torch tensors and torch's current HIP stream, at the five
configurations' full sizes, against the fp64 oracle. Every other GPU test goes through the
Python binding, which calls rn_forward_ex."""

import ctypes
import os

import pytest
import torch

import oracle
import row_wise_normalization_fp32_amd as rn
import workloads
from _compare import STAT_REL_TOL, check_bits_equal, check_equal_values, check_mean, check_rel, check_rstd, \
    check_softmax_y, check_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS = min(16, os.cpu_count() or 1)
DT = {"fp32": 0, "fp16": 1, "bf16": 2}
LIB = rn._lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _f32(rows):
    return torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)


def _run(w, inp, with_params=True, with_stats=True):
    g = {k: v.to(DEV) for k, v in inp.items()}
    y = torch.full_like(g["x"], float("nan"))
    rows, N, dt = w.rows, w.N, DT[w.dtype]
    par = (lambda k: g.get(k)) if with_params else (lambda k: None)
    out = {"y": y}
    if w.op == "ln":
        mean, rstd = (_f32(rows), _f32(rows)) if with_stats else (None, None)
        st = LIB.ln_forward(_p(g["x"]), _p(par("gamma")), _p(par("beta")), _p(y), _p(mean), _p(rstd), rows, N,
                            ctypes.c_float(w.eps), dt, _stream())
        out.update(mean=mean, rstd=rstd)
    elif w.op == "rms":
        rstd = _f32(rows) if with_stats else None
        st = LIB.rms_norm(_p(g["x"]), _p(par("weight")), _p(y), _p(rstd), rows, N, ctypes.c_float(w.eps), dt,
                          _stream())
        out.update(rstd=rstd)
    elif w.op == "fused_add_rms":
        ro = torch.full_like(g["x"], float("nan"))
        rstd = _f32(rows) if with_stats else None
        st = LIB.fused_add_rms_norm(_p(g["x"]), _p(g["residual"]), _p(par("weight")), _p(y), _p(ro), _p(rstd),
                                    rows, N, ctypes.c_float(w.eps), dt, _stream())
        out.update(residual_out=ro, rstd=rstd)
    elif w.op == "fused_add_ln":
        ro = torch.full_like(g["x"], float("nan"))
        mean, rstd = (_f32(rows), _f32(rows)) if with_stats else (None, None)
        st = LIB.fused_add_layer_norm(_p(g["x"]), _p(g["residual"]), _p(par("gamma")), _p(par("beta")), _p(y),
                                      _p(ro), _p(mean), _p(rstd), rows, N, ctypes.c_float(w.eps), dt, _stream())
        out.update(residual_out=ro, mean=mean, rstd=rstd)
    else:
        mx, sm = (_f32(rows), _f32(rows)) if with_stats else (None, None)
        st = LIB.softmax_forward(_p(g["x"]), _p(y), _p(mx), _p(sm), rows, N, dt, _stream())
        out.update(max=mx, sum=sm)
    torch.cuda.synchronize()
    assert st == 0, rn.STATUS.get(st, st)
    return out


def _oracle(w, inp):
    if w.op == "ln":
        return oracle.layer_norm(inp["x"], inp.get("gamma"), inp.get("beta"), w.eps, threads=THREADS)
    if w.op == "rms":
        return oracle.rms_norm(inp["x"], inp.get("weight"), w.eps, threads=THREADS)
    if w.op == "fused_add_rms":
        return oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp.get("weight"), w.eps, threads=THREADS)
    if w.op == "fused_add_ln":
        return oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp.get("gamma"), inp.get("beta"), w.eps,
                                           threads=THREADS)
    return oracle.softmax(inp["x"], threads=THREADS)


def _check(w, ref, out, with_stats=True):
    if w.op == "softmax":
        check_softmax_y(out["y"], ref["y"])
        if with_stats:
            check_equal_values(out["max"], ref["max"], "row_max")
            check_rel(out["sum"], ref["sum"], STAT_REL_TOL, "row_sum")
        return
    check_y(out["y"], ref["y"], "y", op=w.op)
    if w.op in ("fused_add_rms", "fused_add_ln"):
        check_bits_equal(out["residual_out"], ref["residual_out"], "residual_out")
    if with_stats:
        if w.op in ("ln", "fused_add_ln"):
            check_mean(out["mean"], ref["mean"], ref["rstd"], w.eps)
        check_rstd(out["rstd"], ref["rstd"])


@pytest.mark.parametrize("w", workloads.CONFIGS, ids=[c.name for c in workloads.CONFIGS])
def test_plain_entry_point_full_size(w):
    inp = workloads.make_inputs(w)
    _check(w, _oracle(w, inp), _run(w, inp))


@pytest.mark.parametrize("w", [workloads.FUSED_LN, workloads.SOFTMAX, workloads.C4_BF16.scaled(rows=2048),
                               workloads.C5.scaled(rows=2048, N=4096)], ids=lambda w: f"{w.op}_{w.rows}x{w.N}")
def test_plain_entry_point_other_ops_and_8m(w):
    inp = workloads.make_inputs(w)
    _check(w, _oracle(w, inp), _run(w, inp))


@pytest.mark.parametrize("w", [workloads.C1, workloads.C3, workloads.C4_FP16, workloads.FUSED_LN],
                         ids=lambda w: w.name)
def test_plain_entry_point_without_parameters_and_statistics(w):
    # the nullable arguments: parameters absent (gamma = 1, beta = 0, weight = 1), no statistics
    w = w.scaled(rows=96, with_gamma=False, with_beta=False)
    inp = workloads.make_inputs(w)
    _check(w, _oracle(w, inp), _run(w, inp, with_params=False, with_stats=False), with_stats=False)
