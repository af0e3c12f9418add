"""GPU parity of caller-chosen launch plans (rn_forward_tuned through the binding's
``tuning=``): every built alternative of a shape's plan meets the fp64 oracle, and the ones
that keep the automatic row-group shape (waves and chunks per lane) and change only the
launch (grid per row or persistent, prefetching or looping instance, grid size) give the
automatic plan's results bit for bit. Row counts are chosen so that grids of a few
workgroups loop over many rows, with a ragged last round."""

import os

import pytest
import torch

import oracle
import row_wise_normalization_fp32_amd as rn
import workloads
from _compare import check_bits_equal, check_equal_values, check_mean, check_rel, check_rstd, check_softmax_y, \
    check_y, STAT_REL_TOL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS = min(16, os.cpu_count() or 1)

SHAPES = [
    workloads.C5.scaled(rows=301, N=4096, seed=1701, name="ln_bf16_301x4096"),
    workloads.C5.scaled(rows=67, N=16384, seed=1702, name="ln_bf16_67x16384"),
    workloads.C3.scaled(rows=259, seed=1703, name="rms_fp16_259x4096"),
    workloads.C4_FP16.scaled(rows=263, seed=1704, name="fused_fp16_263x4096"),
    workloads.FUSED_LN.scaled(rows=131, N=8192, seed=1705, name="fused_ln_bf16_131x8192"),
    workloads.SOFTMAX.scaled(rows=270, seed=1706, name="softmax_fp32_270x4096"),
    workloads.C1.scaled(rows=517, seed=1707, name="ln_fp32_517x1024"),
    # rows held exactly by 3, 5 or 7 chunks per lane (2 waves x 5, 4 x 3, 4 x 7)
    workloads.C5.scaled(rows=523, N=5120, seed=1708, name="ln_bf16_523x5120"),
    workloads.FUSED_LN.scaled(rows=263, N=6144, seed=1709, name="fused_ln_bf16_263x6144"),
    workloads.C3.scaled(rows=259, N=14336, seed=1710, name="rms_fp16_259x14336"),
    # byte-addressed rows (2 and 8 waves), launch tunings only
    workloads.C5.scaled(rows=523, N=4095, seed=1711, name="ln_bf16_523x4095"),
    workloads.C5.scaled(rows=263, N=16383, seed=1712, name="ln_bf16_263x16383"),
]

TUNINGS = ([{"waves_per_row": w} for w in (1, 2, 4, 8, 16)] +
           [{"waves_per_row": w, "persistent": p} for w in (1, 2, 4, 8, 16) for p in (0, 1)] +
           [{"persistent": 1, "prefetch": pf, "grid_blocks": g} for pf in (0, 1) for g in (1, 7, 64, 100000)] +
           [{"persistent": 0, "grid_blocks": g} for g in (1, 5)])


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


def _run(w, g, tuning):
    kw = {} if tuning is None else {"tuning": tuning}
    if w.op == "ln":
        y, m, r = rn.ln_forward(g["x"], g["gamma"], g["beta"], w.eps, return_stats=True, **kw)
        return {"y": y, "mean": m, "rstd": r}
    if w.op == "rms":
        y, r = rn.rms_norm(g["x"], g["weight"], w.eps, return_rstd=True, **kw)
        return {"y": y, "rstd": r}
    if w.op == "fused_add_rms":
        y, ro, r = rn.fused_add_rms_norm(g["x"], g["residual"], g["weight"], w.eps, return_rstd=True, **kw)
        return {"y": y, "residual_out": ro, "rstd": r}
    if w.op == "fused_add_ln":
        y, ro, m, r = rn.fused_add_layer_norm(g["x"], g["residual"], g["gamma"], g["beta"], w.eps,
                                              return_stats=True, **kw)
        return {"y": y, "residual_out": ro, "mean": m, "rstd": r}
    y, mx, sm = rn.softmax_forward(g["x"], return_stats=True, **kw)
    return {"y": y, "max": mx, "sum": sm}


def _check_oracle(w, ref, o):
    if w.op == "softmax":
        check_softmax_y(o["y"], ref["y"])
        check_equal_values(o["max"], ref["max"], "row_max")
        check_rel(o["sum"], ref["sum"], STAT_REL_TOL, "row_sum")
        return
    check_y(o["y"], ref["y"], "y", op=w.op)
    check_rstd(o["rstd"], ref["rstd"])
    if "mean" in o:
        check_mean(o["mean"], ref["mean"], ref["rstd"], w.eps)
    if "residual_out" in o:
        check_bits_equal(o["residual_out"], ref["residual_out"], "residual_out")


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_every_built_plan_meets_the_oracle(w):
    inp = workloads.make_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    ref = _oracle(w, inp)
    ptrs = {k: g[k].data_ptr() for k in ("x", "residual", "gamma", "beta", "weight") if k in g}
    if "weight" in ptrs:
        ptrs["gamma"] = ptrs.pop("weight")
    td = workloads.TORCH_DTYPES[w.dtype]
    st, auto = rn.plan(w.op, w.rows, w.N, td, ptrs=ptrs, eps=w.eps)
    assert st == 0
    base = _run(w, g, None)
    torch.cuda.synchronize()
    _check_oracle(w, ref, base)
    ran = 0
    for t in TUNINGS:
        st, info = rn.plan(w.op, w.rows, w.N, td, ptrs=ptrs, eps=w.eps, tuning=t)
        if st != 0:
            continue  # not built for this shape (rn_plan_tuned says so on the host)
        o = _run(w, g, t)
        torch.cuda.synchronize()
        print(f"{w.name} tuning {t}: W{info['waves_per_row']} V{info['chunks_per_lane']} "
              f"persistent={info['persistent']} grid={info['grid_blocks']}", flush=True)
        _check_oracle(w, ref, o)
        if (info["waves_per_row"], info["chunks_per_lane"]) == (auto["waves_per_row"], auto["chunks_per_lane"]):
            for k in base:
                assert torch.equal(_bits(o[k]), _bits(base[k])), (t, k)
        ran += 1
    assert ran >= 6, ran
