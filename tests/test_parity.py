"""GPU parity: the HIP library against the fp64 oracle, element by element.

Every call goes through the C ABI (via the ctypes binding). Inputs come from the seeded
generators in workloads.py; expected values come only from the oracle. Tolerances are
stated in tests/_compare.py.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import row_wise_normalization_fp32_amd as rn
import workloads
from _compare import (STAT_REL_TOL, check_bits_equal, check_equal_values, check_mean, check_rel, check_rstd,
                      check_softmax_y, check_y, dtype_name)

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)
DEV = "cuda:0"
TD = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def _gpu(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def run_gpu(w: workloads.Workload, inp, variant="auto", stats=True):
    """Returns (y, second, third, fourth): LayerNorm (y, mean, rstd, None); RMSNorm (y, None,
    rstd, None); fused add + RMSNorm (y, residual_out, rstd, None); fused add + LayerNorm
    (y, residual_out, rstd, mean); softmax (y, None, row_sum, row_max)."""
    g = _gpu(inp)
    if w.op == "ln":
        out = rn.ln_forward(g["x"], g.get("gamma"), g.get("beta"), w.eps, return_stats=stats, variant=variant)
        return (out + (None,)) if stats else (out, None, None, None)
    if w.op == "rms":
        y, rstd = rn.rms_norm(g["x"], g.get("weight"), w.eps, return_rstd=True, variant=variant)
        return y, None, rstd, None
    if w.op == "fused_add_ln":
        y, ro, mean, rstd = rn.fused_add_layer_norm(g["x"], g["residual"], g.get("gamma"), g.get("beta"), w.eps,
                                                    return_stats=True, variant=variant)
        return y, ro, rstd, mean
    if w.op == "softmax":
        y, mx, sm = rn.softmax_forward(g["x"], return_stats=True, variant=variant)
        return y, None, sm, mx
    y, ro, rstd = rn.fused_add_rms_norm(g["x"], g["residual"], g.get("weight"), w.eps, return_rstd=True,
                                        variant=variant)
    return y, ro, rstd, None


def run_oracle(w: workloads.Workload, inp):
    if w.op == "ln":
        return oracle.layer_norm(inp["x"], inp.get("gamma"), inp.get("beta"), w.eps, threads=THREADS)
    if w.op == "rms":
        return oracle.rms_norm(inp["x"], inp.get("weight"), w.eps, threads=THREADS)
    if w.op == "fused_add_ln":
        return oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp.get("gamma"), inp.get("beta"), w.eps,
                                           threads=THREADS)
    if w.op == "softmax":
        return oracle.softmax(inp["x"], threads=THREADS)
    return oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp.get("weight"), w.eps, threads=THREADS)


def check_outputs(w: workloads.Workload, ref, a, b, c, d):
    if w.op == "softmax":
        err = check_softmax_y(a, ref["y"])
        check_equal_values(d, ref["max"], "row_max")
        check_rel(c, ref["sum"], STAT_REL_TOL, "row_sum")
        return err
    err = check_y(a, ref["y"], op=w.op)
    if w.op == "ln":
        check_mean(b, ref["mean"], ref["rstd"], w.eps)
        check_rstd(c, ref["rstd"])
    elif w.op == "rms":
        check_rstd(c, ref["rstd"])
    elif w.op == "fused_add_ln":
        check_bits_equal(b, ref["residual_out"], "residual_out")
        check_mean(d, ref["mean"], ref["rstd"], w.eps)
        check_rstd(c, ref["rstd"])
    else:
        check_bits_equal(b, ref["residual_out"], "residual_out")
        check_rstd(c, ref["rstd"])
    return err


def check_case(w: workloads.Workload, variant="auto", inp=None):
    inp = workloads.make_inputs(w) if inp is None else inp
    ref = run_oracle(w, inp)
    a, b, c, d = run_gpu(w, inp, variant)
    torch.cuda.synchronize()
    return check_outputs(w, ref, a, b, c, d)


# ---------------------------------------------------------------------------------------
# The six headline configurations at full size, in the launch configuration the
# benchmark times (automatic variant choice).
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("w", workloads.CONFIGS, ids=[c.name for c in workloads.CONFIGS])
def test_config_full_size(w):
    check_case(w)


def test_fused_large_shape():
    check_case(workloads.FUSED_8192)


@pytest.mark.parametrize("w", [workloads.FUSED_LN, workloads.FUSED_LN_8192, workloads.SOFTMAX,
                               workloads.SOFTMAX_8192], ids=lambda w: w.name)
def test_new_ops_full_size(w):
    check_case(w)


@pytest.mark.parametrize("w,variant", [(workloads.LN_RAGGED, "workgroup"), (workloads.LN_SPLIT, "wide"),
                                       (workloads.SOFTMAX_VOCAB, "workgroup")], ids=lambda v: getattr(v, "name", v))
def test_general_shapes_full_size(w, variant):
    # the benchmark's general-shape workloads at full size, in the launch configuration it
    # times (automatic choice; the binding supplies the split-row workspace)
    td = TD[w.dtype]
    st, info = rn.plan(w.op, w.rows, w.N, td, workspace_bytes=rn.forward_workspace_bytes(w.op, w.rows, w.N, td))
    assert st == 0 and info["variant"] == variant, info
    check_case(w)


# ---------------------------------------------------------------------------------------
# Every kernel variant on shapes spanning several tiles and a ragged tail.
# ---------------------------------------------------------------------------------------

SHAPES = [(37, 1000), (5, 4096), (9, 2056), (3, 8)]


BASES = {"ln": workloads.C1, "rms": workloads.C3, "fused_add_rms": workloads.C4_FP16,
         "fused_add_ln": workloads.FUSED_LN, "softmax": workloads.SOFTMAX}


@pytest.mark.parametrize("variant", ["wave", "workgroup", "element", "general"])
@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_variants_agree_with_oracle(variant, op, dtype):
    base = BASES[op]
    for rows, N in SHAPES:
        w = base.scaled(rows=rows, N=N, seed=500 + rows, dtype=dtype)
        check_case(w, variant)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_workgroup_path_long_rows(dtype):
    for rows, N in [(7, 16384), (6, 12296), (4, 8200)]:
        check_case(workloads.C5.scaled(rows=rows, N=N, seed=600 + N, dtype=dtype))


def test_workgroup_path_32k_bf16_rows():
    check_case(workloads.C5.scaled(rows=5, N=32768, seed=601))


WIDE_SHAPES = {"fp32": [(3, 32772), (2, 40960), (3, 65536)], "bf16": [(3, 65544), (2, 131080)],
               "fp16": [(3, 81920)]}
BIG_SHAPES = {"fp32": [(3, 16388), (4, 24576), (2, 32768)], "bf16": [(3, 32776), (2, 65536)], "fp16": [(3, 40960)]}


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_workgroup_path_128k_rows(op, dtype):
    # rows of 64-128 KiB: softmax, RMSNorm and LayerNorm in one 16-wave workgroup holding 8
    # chunks per lane (x read once); the fused ops take the split-row path there
    for rows, N in BIG_SHAPES[dtype]:
        td = TD[dtype]
        st, info = rn.plan(op, rows, N, td, workspace_bytes=rn.forward_workspace_bytes(op, rows, N, td))
        if op in ("softmax", "rms", "ln"):
            assert st == 0 and info["variant"] == "workgroup" and info["chunks_per_lane"] == 8, info
        else:
            assert st == 0 and info["variant"] == "wide", info
        check_case(BASES[op].scaled(rows=rows, N=N, seed=680 + N, dtype=dtype))


@pytest.mark.parametrize("op", ["ln", "fused_add_rms"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_workgroup_path_128k_rows_without_workspace(op, dtype):
    # without a workspace (C callers that pass none; here a forced variant, for which the
    # binding allocates none) LayerNorm and fused add + RMSNorm rows of 64-128 KiB take one
    # 16-wave workgroup with 8 chunks per lane instead of the general kernel
    for rows, N in BIG_SHAPES[dtype]:
        st, info = rn.plan(op, rows, N, TD[dtype], variant="workgroup")
        assert st == 0 and info["chunks_per_lane"] == 8 and info["waves_per_row"] == 16, info
        check_case(BASES[op].scaled(rows=rows, N=N, seed=690 + N, dtype=dtype), variant="workgroup")


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_split_rows(op, dtype):
    # rows longer than a workgroup's registers: statistics per 32 KiB segment, then a
    # fixed-order combine in every segment's workgroup (the binding passes a workspace)
    for rows, N in WIDE_SHAPES[dtype]:
        st, info = rn.plan(op, rows, N, TD[dtype], workspace_bytes=rn.forward_workspace_bytes(op, rows, N, TD[dtype]))
        # (fp32 softmax rows of up to 65536 elements stay in one workgroup, 16 chunks per lane)
        expect = "workgroup" if op == "softmax" and dtype == "fp32" and N <= 65536 else "wide"
        assert st == 0 and info["variant"] == expect, info
        check_case(BASES[op].scaled(rows=rows, N=N, seed=620 + N, dtype=dtype))


ELEM_WIDE_SHAPES = {"fp32": [(3, 16385), (2, 50257), (3, 65537)], "bf16": [(3, 20001), (2, 50257), (2, 131073)],
                    "fp16": [(3, 32769)]}


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_split_rows_element(op, dtype):
    # rows of more than 16384 elements that are not whole 16-byte chunks (a vocabulary-sized
    # softmax, 50257): by default byte-addressed one-pass segments; forced, statistics per
    # 8192-element segment, then the same fixed-order combine (softmax rows of up to 65536
    # elements stay in one workgroup: byte-addressed 16-wave rows beyond 4096 chunks, else the
    # element / pair kernels)
    for rows, N in ELEM_WIDE_SHAPES[dtype]:
        st, info = rn.plan(op, rows, N, TD[dtype], workspace_bytes=rn.forward_workspace_bytes(op, rows, N, TD[dtype]))
        # (these 16-bit rows have odd lengths: at odd 2-byte positions, element segments)
        chunks = -(-N * (4 if dtype == "fp32" else 2) // 16)
        if op == "softmax" and N <= 65536:
            expect = "workgroup" if chunks > 4096 else "element"
        else:
            expect = "wide" if dtype == "fp32" else "wide_element"
        assert st == 0 and info["variant"] == expect, info
        check_case(BASES[op].scaled(rows=rows, N=N, seed=660 + N, dtype=dtype))
        if expect == "wide":
            check_case(BASES[op].scaled(rows=rows, N=N, seed=660 + N, dtype=dtype), "wide_element")
    # forced on rows of whole chunks (segments end exactly on the row's end)
    check_case(BASES[op].scaled(rows=2, N=65536, seed=661, dtype=dtype), "wide_element")


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_softmax_long_rows_one_workgroup(dtype):
    # softmax rows of 16385-65536 elements that are not whole chunks (or unaligned): one
    # 16-wave workgroup per row, byte-addressed 16-byte chunks beyond 4096 chunks (8 per lane,
    # fp32 up to 16), else the element / pair kernels; forced, the element / pair kernels
    # holding up to 64 elements (32 pairs) per lane
    for rows, N, v in [(3, 16385, 32), (2, 32768 + 7, 64), (2, 50257, 64), (2, 65535, 64)]:
        td = TD[dtype]
        esz = 4 if dtype == "fp32" else 2
        chunks = -(-N * esz // 16)
        st, info = rn.plan("softmax", rows, N, td, workspace_bytes=rn.forward_workspace_bytes("softmax", rows, N, td))
        assert st == 0 and info["waves_per_row"] == 16, info
        if chunks > 4096:
            assert info["variant"] == "workgroup" and info["ragged"], info
            assert info["chunks_per_lane"] == (8 if chunks <= 8192 else 16), info
        else:
            assert info["variant"] == "element", info
        w = workloads.SOFTMAX.scaled(rows=rows, N=N, seed=690 + N, dtype=dtype)
        check_case(w)
        st, info = rn.plan("softmax", rows, N, td, variant="element")
        assert st == 0 and info["variant"] == "element" and info["waves_per_row"] == 16, info
        assert info["chunks_per_lane"] == (v if dtype == "fp32" else v // 2) and info["pairs"] == (dtype != "fp32")
        check_case(w, "element")
    # large logits (spread +-160) on the longest rows
    check_case(workloads.SOFTMAX.scaled(rows=2, N=65535, seed=699, dtype="fp32", x_scale=80.0))
    if dtype == "fp32":
        # whole-chunk fp32 rows of up to 65536 elements: 16 chunks per lane
        for rows, N in [(3, 40960), (2, 50304), (2, 65536)]:
            st, info = rn.plan("softmax", rows, N, torch.float32)
            assert st == 0 and info["variant"] == "workgroup" and info["chunks_per_lane"] == 16, info
            check_case(workloads.SOFTMAX.scaled(rows=rows, N=N, seed=695 + N))


def test_split_rows_element_offsets_strides_constant_and_in_place():
    # cancellation stress, constant rows, unaligned and padded rows, NaN guards, in place
    check_case(workloads.C2.scaled(rows=4, N=65537, seed=670))
    w = workloads.C2.scaled(rows=3, N=50257, seed=671, x_dist="constant")
    g = _gpu(workloads.make_inputs(w))
    y = rn.ln_forward(g["x"], g["gamma"], g["beta"], w.eps)
    torch.cuda.synchronize()
    assert torch.equal(y, g["beta"].expand_as(y))
    for op in ("ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"):
        w = BASES[op].scaled(rows=3, N=20001, seed=672, dtype="bf16")
        inp = workloads.make_inputs(w)
        ref = run_oracle(w, inp)
        for off, ld in [({n: 1 for n in ROW_TENSORS}, None), ({"x": 3, "y": 0}, {n: 20003 for n in ROW_TENSORS})]:
            out = run_placed(w, inp, offset=off, ld=ld, expect_variant="element" if op == "softmax" else "wide_element")
            check_outputs(w, ref, *out)
    w = workloads.C5.scaled(rows=3, N=50257, seed=673)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    x = inp["x"].to(DEV)
    rn.ln_forward(x, inp["gamma"].to(DEV), inp["beta"].to(DEV), w.eps, out=x)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="ln")
    w = workloads.FUSED_LN.scaled(rows=3, N=50257, seed=674)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    rn.fused_add_layer_norm(g["x"], g["residual"], g["gamma"], g["beta"], w.eps, out=g["x"],
                            residual_out=g["residual"])
    torch.cuda.synchronize()
    check_y(g["x"], ref["y"], op="fused_add_ln")
    check_bits_equal(g["residual"], ref["residual_out"], "split-row element residual_out in place")


def test_split_rows_offset_constant_and_in_place():
    # cancellation stress and constant rows on the split-row path
    check_case(workloads.C2.scaled(rows=4, N=65536, seed=630))
    w = workloads.C2.scaled(rows=3, N=65536, seed=631, x_dist="constant")
    g = _gpu(workloads.make_inputs(w))
    y = rn.ln_forward(g["x"], g["gamma"], g["beta"], w.eps)
    torch.cuda.synchronize()
    assert torch.equal(y, g["beta"].expand_as(y))
    # in place: y over x; fused: residual_out over residual and y over x
    w = workloads.C5.scaled(rows=3, N=131072, seed=632)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    x = inp["x"].to(DEV)
    rn.ln_forward(x, inp["gamma"].to(DEV), inp["beta"].to(DEV), w.eps, out=x)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="ln")
    w = workloads.FUSED_LN.scaled(rows=3, N=65536, seed=633)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    rn.fused_add_layer_norm(g["x"], g["residual"], g["gamma"], g["beta"], w.eps, out=g["x"],
                            residual_out=g["residual"])
    torch.cuda.synchronize()
    check_y(g["x"], ref["y"], op="fused_add_ln")
    check_bits_equal(g["residual"], ref["residual_out"], "split-row residual_out in place")


def test_offset_rows_on_every_variant():
    # The cancellation stress (row offsets up to +-1000) on each kernel.
    for variant in ("wave", "workgroup", "general"):
        check_case(workloads.C2.scaled(rows=16, seed=610), variant)
    check_case(workloads.C2.scaled(rows=8, N=16384, seed=611))


# ---------------------------------------------------------------------------------------
# Edge cases.
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 3, 7, 64, 255, 1023, 4097, 8191, 16383, 16385, 20000])
def test_odd_widths(N):
    for op, base in (("ln", workloads.C1), ("rms", workloads.C3), ("fused_add_rms", workloads.C4_BF16),
                     ("fused_add_ln", workloads.FUSED_LN), ("softmax", workloads.SOFTMAX.scaled(dtype="fp16"))):
        check_case(base.scaled(rows=3, N=N, seed=700 + N))


@pytest.mark.parametrize("case", [("ln", "bf16", 16384, 4095, "workgroup"), ("fused_add_ln", "fp16", 8192, 1001, "wave"),
                                  ("rms", "fp32", 16384, 101, "wave"), ("fused_add_rms", "bf16", 2048, 16383, "element"),
                                  ("softmax", "fp32", 16384, 333, "wave")], ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}")
def test_element_kernel_persistent(case):
    # many ragged rows go to the byte-addressed vectorized kernel by default (16-bit fused rows
    # of 8 waves at odd 2-byte positions to the pair kernel); forced, the element / pair kernels
    # run persistent
    op, dtype, rows, N, auto = case
    st, info = rn.plan(op, rows, N, TD[dtype])
    assert st == 0 and info["variant"] == auto and info["ragged"] == (auto != "element"), info
    st, info = rn.plan(op, rows, N, TD[dtype], variant="element")
    assert st == 0 and info["variant"] == "element" and info["persistent"], info
    check_case(BASES[op].scaled(rows=rows, N=N, seed=720 + N, dtype=dtype), "element")


ROW_TENSORS = ("x", "residual", "y", "residual_out")


def run_placed(w: workloads.Workload, inp, offset=None, ld=None, variant="auto", expect_pairs=None,
               expect_variant=None):
    """Runs the op with each row tensor placed in its own NaN-filled buffer, at an element
    offset (``offset[name]``) and row stride (``ld[name]``, default N), with 64 guard
    elements on both sides. Checks that nothing outside the outputs' rows is written and,
    if ``expect_pairs`` is given, that the plan for these very pointers agrees. Returns the
    outputs in run_gpu's order (the binding supplies a split-row workspace when one is
    needed)."""
    offset, ld = offset or {}, ld or {}
    g = _gpu(inp)
    rows, N = inp["x"].shape
    T = inp["x"].dtype
    fused = w.op in ("fused_add_rms", "fused_add_ln")
    names = ROW_TENSORS if fused else ("x", "y")
    bufs, views = {}, {}
    for n in names:
        o, l = offset.get(n, 0), ld.get(n, N)
        buf = torch.full((64 + o + (rows - 1) * l + N + 64,), float("nan"), dtype=T, device=DEV)
        views[n] = buf.as_strided((rows, N), (l, 1), 64 + o)
        bufs[n] = buf
        if n in ("x", "residual"):
            views[n].copy_(g[n])
    ptrs = {n: views[n].data_ptr() for n in names}
    strides = {n: ld.get(n, N) for n in names}
    if "gamma" in g:
        ptrs["gamma"] = g["gamma"].data_ptr()
    st, info = rn.plan(w.op, rows, N, T, ptrs=ptrs, strides=strides, variant=variant,
                       workspace_bytes=rn.forward_workspace_bytes(w.op, rows, N, T))
    assert st == 0, st
    if expect_variant is not None:
        assert info["variant"] == expect_variant, info
    if expect_pairs is not None:
        assert info["variant"] == "element" and info["pairs"] == expect_pairs, info
    x, y = views["x"], views["y"]
    if w.op == "ln":
        out = rn.ln_forward(x, g.get("gamma"), g.get("beta"), w.eps, out=y, return_stats=True,
                            variant=variant) + (None,)
    elif w.op == "rms":
        yy, rstd = rn.rms_norm(x, g.get("weight"), w.eps, out=y, return_rstd=True, variant=variant)
        out = (yy, None, rstd, None)
    elif w.op == "fused_add_rms":
        yy, ro, rstd = rn.fused_add_rms_norm(x, views["residual"], g.get("weight"), w.eps, out=y,
                                             residual_out=views["residual_out"], return_rstd=True, variant=variant)
        out = (yy, ro, rstd, None)
    elif w.op == "fused_add_ln":
        yy, ro, mean, rstd = rn.fused_add_layer_norm(x, views["residual"], g.get("gamma"), g.get("beta"), w.eps,
                                                     out=y, residual_out=views["residual_out"], return_stats=True,
                                                     variant=variant)
        out = (yy, ro, rstd, mean)
    else:
        yy, mx, sm = rn.softmax_forward(x, out=y, return_stats=True, variant=variant)
        out = (yy, None, sm, mx)
    torch.cuda.synchronize()
    for n in ("y", "residual_out"):
        if n not in views:
            continue
        inside = torch.zeros(bufs[n].shape, dtype=torch.bool, device=DEV)
        inside.as_strided((rows, N), (strides[n], 1), 64 + offset.get(n, 0)).fill_(True)
        assert torch.isnan(bufs[n][~inside]).all(), f"{n}: written outside its rows"
    return out


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
def test_element_kernel_every_width(op):
    # the element kernel's (W, V) instances: W = 1 with V = 1..8, W = 2..16 with V = 8, W = 16 with V = 16;
    # 16-bit rows take it when their tensors sit at different positions in 4-byte words
    # (here: x one element off), else they move as element pairs
    for rows, N in [(5, 33), (4, 100), (3, 300), (6, 511), (5, 1000), (3, 2047), (2, 4093), (2, 8191),
                    (2, 12289), (2, 16384)]:
        check_case(BASES[op].scaled(rows=rows, N=N, seed=710 + N, dtype="fp32"), "element")
        w = BASES[op].scaled(rows=rows, N=N, seed=710 + N, dtype="bf16")
        inp = workloads.make_inputs(w)
        out = run_placed(w, inp, offset={"x": 1}, variant="element", expect_pairs=False)
        check_outputs(w, run_oracle(w, inp), *out)


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_pair_kernel_every_width(op, dtype):
    # the pair kernel's (W, V) instances: W = 1 with V = 1, 2, 4, 8; W = 2, 4, 8, 16 with V = 8.
    # Odd N: every other row starts in the upper half of a 4-byte word.
    for rows, N in [(5, 33), (4, 201), (3, 301), (6, 1001), (3, 1002), (5, 2045), (3, 4093), (3, 4094),
                    (2, 8191), (2, 12289), (2, 16383)]:
        w = BASES[op].scaled(rows=rows, N=N, seed=740 + N, dtype=dtype)
        assert rn.plan(op, rows, N, TD[dtype])[1]["pairs"]
        check_case(w)
    # 16384 elements whose rows all start on a word: exactly the 8192 words of W = 16, V = 8
    w = BASES[op].scaled(rows=3, N=16384, seed=741, dtype=dtype)
    assert rn.plan(op, 3, 16384, TD[dtype], variant="element")[1]["pairs"]
    check_case(w, "element")


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
def test_pair_kernel_offsets_strides_and_guards(op):
    # rows starting in the upper half of a word from row 0 on, odd and even strides; nothing
    # outside the output rows written (NaN guards); mismatched tensors fall back to single
    # elements
    for N in (33, 1000, 4095):
        w = BASES[op].scaled(rows=7, N=N, seed=750 + N, dtype="bf16")
        inp = workloads.make_inputs(w)
        ref = run_oracle(w, inp)
        all_one = {n: 1 for n in ROW_TENSORS}
        cases = [
            (all_one, None, True),
            ({"x": 3, "y": 1, "residual": 5, "residual_out": 7}, None, True),
            (None, {n: N + 1 for n in ROW_TENSORS}, True),
            (all_one, {"x": N + 3, "y": N + 1, "residual": N + 5, "residual_out": N + 1}, True),
            ({"y": 1}, None, False),
            (None, {"x": N + 1, "y": N + 2}, False),
        ]
        for off, ld, pairs in cases:
            out = run_placed(w, inp, offset=off, ld=ld, expect_pairs=pairs)
            check_outputs(w, ref, *out)


def test_zero_rows_is_a_noop():
    x = torch.empty(0, 64, device=DEV)
    y = rn.ln_forward(x)
    assert y.shape == (0, 64)
    y, ro = rn.fused_add_rms_norm(x, x.clone())
    assert ro.shape == (0, 64)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_optional_parameters(dtype):
    for with_g, with_b in [(False, False), (True, False), (False, True)]:
        w = workloads.C1.scaled(rows=9, N=1024, seed=800, dtype=dtype, with_gamma=with_g, with_beta=with_b)
        for variant in ("wave", "workgroup", "general"):
            check_case(w, variant)
    w = workloads.C3.scaled(rows=9, N=512, seed=801, dtype=dtype, with_gamma=False)
    check_case(w)
    w = workloads.C4_FP16.scaled(rows=9, N=512, seed=802, dtype=dtype, with_gamma=False)
    check_case(w)


def test_constant_rows_map_to_beta():
    for dtype in ("fp32", "fp16", "bf16"):
        for N in (1024, 16384):
            w = workloads.C2.scaled(rows=6, N=N, seed=810, dtype=dtype, x_dist="constant")
            inp = workloads.make_inputs(w)
            g = _gpu(inp)
            y, mean, rstd = rn.ln_forward(g["x"], g["gamma"], g["beta"], w.eps, return_stats=True)
            torch.cuda.synchronize()
            beta = g["beta"].expand_as(y)
            assert torch.equal(y, beta), f"{dtype} N={N}: constant rows must give beta exactly"
            assert torch.equal(mean, g["x"][:, 0].float())


def test_misaligned_pointers_use_element_path():
    w = workloads.C1.scaled(rows=5, N=1024, seed=820)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    buf = torch.empty(5 * 1024 + 1, device=DEV)
    x = buf[1:].view(5, 1024)
    x.copy_(inp["x"].to(DEV))
    st, info = rn.plan("ln", 5, 1024, torch.float32, ptrs={"x": x.data_ptr()})
    assert info["variant"] == "element"
    y, mean, rstd = rn.ln_forward(x, inp["gamma"].to(DEV), inp["beta"].to(DEV), w.eps, return_stats=True)
    torch.cuda.synchronize()
    check_y(y, ref["y"], op="ln")
    check_rstd(rstd, ref["rstd"])


@pytest.mark.parametrize("variant", ["wave", "workgroup", "element", "general"])
def test_in_place(variant):
    w = workloads.C1.scaled(rows=11, N=2048, seed=830, dtype="bf16")
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    x = g["x"].clone()
    y = rn.ln_forward(x, g["gamma"], g["beta"], w.eps, out=x, variant=variant)
    torch.cuda.synchronize()
    assert y.data_ptr() == x.data_ptr()
    check_y(x, ref["y"], op="ln")
    # fused: residual_out written over residual, y over x
    w = workloads.C4_BF16.scaled(rows=11, N=2048, seed=831)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    x, r = g["x"].clone(), g["residual"].clone()
    rn.fused_add_rms_norm(x, r, g["weight"], w.eps, out=x, residual_out=r, variant=variant)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="fused_add_rms")
    check_bits_equal(r, ref["residual_out"], "residual_out in place")
    # fused: residual_out written over x, y over residual
    x, r = g["x"].clone(), g["residual"].clone()
    rn.fused_add_rms_norm(x, r, g["weight"], w.eps, out=r, residual_out=x, variant=variant)
    torch.cuda.synchronize()
    check_y(r, ref["y"], op="fused_add_rms")
    check_bits_equal(x, ref["residual_out"], "residual_out over x")
    # fused LayerNorm: every pairing of the outputs with the inputs
    w = workloads.FUSED_LN.scaled(rows=11, N=2048, seed=832)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    for y_on, ro_on in (("x", "residual"), ("residual", "x")):
        t = {"x": g["x"].clone(), "residual": g["residual"].clone()}
        rn.fused_add_layer_norm(t["x"], t["residual"], g["gamma"], g["beta"], w.eps, out=t[y_on],
                                residual_out=t[ro_on], variant=variant)
        torch.cuda.synchronize()
        check_y(t[y_on], ref["y"], op="fused_add_ln")
        check_bits_equal(t[ro_on], ref["residual_out"], f"fused LN residual_out over {ro_on}")
    # softmax in place
    w = workloads.SOFTMAX.scaled(rows=11, N=2048, seed=833, dtype="bf16")
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    x = inp["x"].to(DEV)
    rn.softmax_forward(x, out=x, variant=variant)
    torch.cuda.synchronize()
    check_softmax_y(x, ref["y"])


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("pad", [64, 8, 1])
def test_padded_rows(op, pad):
    # x, residual, y and residual_out are column slices of wider buffers (row stride N + pad
    # elements); with bf16, pads 64 and 8 keep rows on 16-byte boundaries (vectorized
    # kernels), pad 1 does not (element kernel). Columns beyond N must not be touched.
    rows, N = 33, 4096
    w = BASES[op].scaled(rows=rows, N=N, seed=860 + pad, dtype="bf16")
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    ld = N + pad

    def slab(src=None):
        buf = torch.full((rows, ld), float("nan"), dtype=torch.bfloat16, device=DEV)
        if src is not None:
            buf[:, :N].copy_(src)
        return buf, buf[:, :N]

    xb, x = slab(g["x"])
    yb, y = slab()
    assert x.stride(0) == ld
    if op in ("fused_add_rms", "fused_add_ln"):
        rb, r = slab(g["residual"])
        ob, ro = slab()
    st, info = rn.plan(op, rows, N, torch.bfloat16, strides={"x": ld, "y": ld, "residual": ld, "residual_out": ld},
                       ptrs={"gamma": 1 << 44, "beta": (1 << 44) + (1 << 30)})
    assert st == 0 and info["variant"] == ("workgroup" if pad % 8 == 0 else "element"), info
    if op == "ln":
        out = rn.ln_forward(x, g["gamma"], g["beta"], w.eps, out=y, return_stats=True) + (None,)
    elif op == "rms":
        yy, rstd = rn.rms_norm(x, g["weight"], w.eps, out=y, return_rstd=True)
        out = (yy, None, rstd, None)
    elif op == "fused_add_rms":
        yy, roo, rstd = rn.fused_add_rms_norm(x, r, g["weight"], w.eps, out=y, residual_out=ro, return_rstd=True)
        out = (yy, roo, rstd, None)
    elif op == "fused_add_ln":
        yy, roo, mean, rstd = rn.fused_add_layer_norm(x, r, g["gamma"], g["beta"], w.eps, out=y, residual_out=ro,
                                                      return_stats=True)
        out = (yy, roo, rstd, mean)
    else:
        yy, mx, sm = rn.softmax_forward(x, out=y, return_stats=True)
        out = (yy, None, sm, mx)
    torch.cuda.synchronize()
    assert out[0].data_ptr() == y.data_ptr()
    check_outputs(w, ref, *out)
    assert torch.isnan(yb[:, N:]).all(), "y padding written"
    if op in ("fused_add_rms", "fused_add_ln"):
        assert torch.isnan(ob[:, N:]).all(), "residual_out padding written"


def test_three_dimensional_input():
    w = workloads.C3.scaled(rows=24, N=4096, seed=840)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    x3 = inp["x"].view(4, 6, 4096).to(DEV)
    y = rn.rms_norm(x3, inp["weight"].to(DEV), w.eps)
    torch.cuda.synchronize()
    assert y.shape == (4, 6, 4096)
    check_y(y.view(24, 4096), ref["y"], op="rms")


def test_outputs_fully_written_and_nothing_outside():
    # Outputs are carved from a NaN-filled buffer with guard zones on both sides.
    for variant in ("wave", "workgroup", "general"):
        w = workloads.C4_FP16.scaled(rows=13, N=1000, seed=850)
        inp = workloads.make_inputs(w)
        g = _gpu(inp)
        n = 13 * 1000
        pad = 4096
        buf = torch.full((2 * n + 3 * pad,), float("nan"), dtype=torch.float16, device=DEV)
        y = buf[pad:pad + n].view(13, 1000)
        ro = buf[2 * pad + n:2 * pad + 2 * n].view(13, 1000)
        rstd = torch.full((13 + 2 * 64,), float("nan"), device=DEV)
        rn.fused_add_rms_norm(g["x"], g["residual"], g["weight"], w.eps, out=y, residual_out=ro,
                              rstd=rstd[64:64 + 13], variant=variant)
        torch.cuda.synchronize()
        assert not torch.isnan(y).any() and not torch.isnan(ro).any()
        assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[pad + n:2 * pad + n]).all()
        assert torch.isnan(buf[2 * pad + 2 * n:]).all()
        assert torch.isnan(rstd[:64]).all() and torch.isnan(rstd[64 + 13:]).all()
        assert not torch.isnan(rstd[64:64 + 13]).any()


def test_bitwise_deterministic_across_launches():
    for w in (workloads.C2, workloads.C4_BF16, workloads.C5.scaled(rows=64)):
        g = _gpu(workloads.make_inputs(w))
        first = None
        for _ in range(20):
            outs = run_gpu(w, {k: v for k, v in g.items()})
            torch.cuda.synchronize()
            outs = [o.clone() for o in outs if o is not None]
            if first is None:
                first = outs
            else:
                for a, b in zip(first, outs):
                    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_argument_errors_reach_python():
    x = torch.zeros(4, 64, device=DEV)
    with pytest.raises(rn.RowNormError) as e:
        rn.ln_forward(x, out=x[:, :64].clone().view(4, 64), eps=-1.0)
    assert e.value.status == 2
    with pytest.raises(rn.RowNormError) as e:
        rn.ln_forward(torch.zeros(4, 8192, device=DEV), variant="wave")
    assert e.value.status == 5


# ---------------------------------------------------------------------------------------
# Persistent launches: parameters staged on chip once per workgroup, workgroups looping
# over many rows. Shapes chosen to have at least 2048 row-group workgroups at every
# row-group width (1, 2, 4, 8, 16 wavefronts per row).
# ---------------------------------------------------------------------------------------

PERSISTENT_CASES = [
    # (base, dtype, rows, N, with_gamma, with_beta)
    ("ln", "fp32", 8192, 256, True, True),      # 1 wave per row
    ("ln", "fp32", 8192, 256, True, False),
    ("ln", "fp32", 8192, 256, False, True),
    ("ln", "bf16", 4096, 4096, True, True),     # 2 waves per row
    ("ln", "fp32", 2048, 4096, True, True),     # 4 waves per row
    ("ln", "bf16", 2048, 16384, True, False),   # 8 waves per row
    ("ln", "fp32", 2048, 16384, False, True),   # 16 waves per row
    ("ln", "fp16", 2048, 32768, True, True),    # 16 waves per row, 16-bit
    ("rms", "fp16", 8192, 512, True, True),
    ("rms", "bf16", 4096, 8192, True, True),
    ("fused_add_rms", "bf16", 4096, 4096, True, True),
    ("fused_add_rms", "fp32", 8192, 2048, True, True),
    ("fused_add_ln", "bf16", 8192, 4096, True, True),
    ("fused_add_ln", "fp16", 2048, 16384, True, False),
    ("fused_add_ln", "fp32", 2048, 16384, False, True),
    ("ln", "bf16", 4096, 16384, False, False),  # no parameters: nothing staged
    ("rms", "fp16", 8192, 4096, False, False),
    ("softmax", "fp32", 8192, 4096, False, False),
    ("softmax", "bf16", 8192, 1024, False, False),  # one wave per row
    ("softmax", "fp16", 4096, 16384, False, False),
]


@pytest.mark.parametrize("case", PERSISTENT_CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-g{int(c[4])}b{int(c[5])}"
                                                        for c in PERSISTENT_CASES])
def test_persistent_launches(case):
    op, dtype, rows, N, wg, wb = case
    base = {"ln": workloads.C5, "rms": workloads.C3, "fused_add_rms": workloads.C4_BF16,
            "fused_add_ln": workloads.FUSED_LN, "softmax": workloads.SOFTMAX}[op]
    w = base.scaled(rows=rows, N=N, seed=900 + N, dtype=dtype, with_gamma=wg, with_beta=wb)
    inp = workloads.make_inputs(w)
    ptrs = {}
    if wg:
        ptrs["gamma"] = 1 << 44
    if wb:
        ptrs["beta"] = (1 << 44) + (1 << 30)
    st, info = rn.plan(op, rows, N, TD[dtype], ptrs=ptrs)
    assert st == 0 and info["persistent"], info
    check_case(w, inp=inp)


def test_persistent_constant_rows_map_to_beta():
    for dtype in ("fp32", "bf16"):
        w = workloads.C2.scaled(rows=4096, N=4096, seed=910, dtype=dtype, x_dist="constant")
        inp = workloads.make_inputs(w)
        g = _gpu(inp)
        y, mean, rstd = rn.ln_forward(g["x"], g["gamma"], g["beta"], w.eps, return_stats=True)
        torch.cuda.synchronize()
        assert torch.equal(y, g["beta"].expand_as(y)), dtype
        assert torch.equal(mean, g["x"][:, 0].float())


def test_persistent_in_place():
    w = workloads.C5.scaled(rows=4096, N=4096, seed=920)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    x = g["x"].clone()
    rn.ln_forward(x, g["gamma"], g["beta"], w.eps, out=x)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="ln")
    w = workloads.C4_FP16.scaled(rows=8192, seed=921)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    x, r = g["x"].clone(), g["residual"].clone()
    rn.fused_add_rms_norm(x, r, g["weight"], w.eps, out=x, residual_out=r)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="fused_add_rms")
    check_bits_equal(r, ref["residual_out"], "residual_out in place (persistent)")
    # fused LayerNorm in place over a persistent launch with 2 waves per row
    w = workloads.FUSED_LN.scaled(rows=8192, seed=922)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    g = _gpu(inp)
    x, r = g["x"].clone(), g["residual"].clone()
    rn.fused_add_layer_norm(x, r, g["gamma"], g["beta"], w.eps, out=x, residual_out=r)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="fused_add_ln")
    check_bits_equal(r, ref["residual_out"], "fused LN residual_out in place (persistent)")


def test_softmax_large_logits_and_constant_rows():
    # logits spread over +-80 (exp ratios near the fp32 range), rows with one dominant
    # element, and constant rows (exactly 1/N)
    for dtype in ("fp32", "bf16"):
        w = workloads.SOFTMAX.scaled(rows=64, N=4096, seed=940, dtype=dtype, x_scale=40.0)
        check_case(w)
        w = workloads.SOFTMAX.scaled(rows=16, N=4096, seed=941, dtype=dtype, x_dist="constant", row_offset=50.0)
        inp = workloads.make_inputs(w)
        y = rn.softmax_forward(inp["x"].to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(y, torch.full_like(y, 1.0 / 4096)), dtype


# Masked logits (-inf entries) through every softmax path: random masks, leading and trailing
# runs, a row with one entry left, and a row with none (NaN outputs, max -inf, sum 0).
MASKED = [("fp32", 64, 4096, None), ("bf16", 64, 4096, None), ("fp32", 4096, 4096, None),  # vec, persistent
          ("fp32", 33, 4095, None), ("bf16", 33, 4095, None), ("fp16", 33, 4095, {"x": 1, "y": 1}),  # element / pairs
          ("bf16", 33, 4096, {"x": 1}),  # single elements
          ("fp32", 16, 32768, None), ("fp32", 16, 65536, None), ("bf16", 8, 65536, None),  # one workgroup, 128-256 KiB
          ("fp32", 4, 50257, None), ("bf16", 4, 50257, None),  # element / pair kernel, 16 waves
          ("fp32", 5, 131072, None), ("bf16", 5, 131073, None)]  # split rows (rows 0-4 carry the patterns)


@pytest.mark.parametrize("dtype,rows,N,off", MASKED, ids=lambda v: str(v))
def test_softmax_masked_rows(dtype, rows, N, off):
    w = workloads.SOFTMAX.scaled(rows=rows, N=N, seed=910 + N % 97, dtype=dtype)
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(N + rows)
    mask = rng.random((rows, N)) < 0.3
    mask[0, :] = False
    mask[1, : N // 2] = True
    mask[2, N // 3:] = True
    mask[3, :] = True  # nothing left: no softmax
    mask[4 % rows, :] = True
    mask[4 % rows, N - 1] = False  # one entry left (y = 1 there)
    x = inp["x"].clone()
    x[torch.from_numpy(mask)] = float("-inf")
    inp = dict(inp, x=x)
    ref = run_oracle(w, inp)
    y, _, ssum, smax = run_placed(w, inp, offset=off) if off else run_gpu(w, inp)
    torch.cuda.synchronize()
    dead = mask.all(axis=1)
    live = torch.from_numpy(~dead)
    yg = y.detach().cpu()
    assert torch.isnan(yg[torch.from_numpy(dead)].float()).all(), "rows without a finite entry must be NaN"
    assert (yg[live][torch.from_numpy(mask[~dead])] == 0).all(), "masked entries must be exactly 0"
    check_softmax_y(yg[live], ref["y"][~dead])
    check_equal_values(smax.cpu(), ref["max"], "row_max")  # -inf where nothing is left
    check_rel(ssum.cpu()[live], ref["sum"][~dead], STAT_REL_TOL, "row_sum")
    assert (ssum.cpu()[torch.from_numpy(dead)] == 0).all()


@pytest.mark.parametrize("op", ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"])
@pytest.mark.parametrize("rows,N", [(4096, 4096), (4096, 4095), (4, 65536)])
def test_nonfinite_rows_stay_in_their_rows(op, rows, N):
    # a NaN or +inf in a row makes that row's outputs non-finite and leaves every other row
    # bit for bit as without it (persistent workgroups loop over many rows; split rows
    # exchange records), whatever the path
    w = BASES[op].scaled(rows=rows, N=N, seed=930, dtype="bf16")
    inp = workloads.make_inputs(w)
    clean = [o.clone() if o is not None else None for o in run_gpu(w, inp)]
    bad_rows = [1, rows // 2, rows - 1]
    x = inp["x"].clone()
    x[bad_rows[0], N // 3] = float("nan")
    x[bad_rows[1], 0] = float("inf")
    x[bad_rows[2], N - 1] = float("nan")
    dirty = run_gpu(w, dict(inp, x=x))
    torch.cuda.synchronize()
    keep = torch.ones(rows, dtype=torch.bool)
    keep[bad_rows] = False
    for c, d in zip(clean, dirty):
        if c is None:
            continue
        assert torch.equal(c[keep].view(torch.uint8) if c.dim() > 1 else c[keep].view(torch.uint8),
                           d[keep].view(torch.uint8) if d.dim() > 1 else d[keep].view(torch.uint8))
    y = dirty[0]
    for r in bad_rows:
        assert not torch.isfinite(y[r].float()).all()
