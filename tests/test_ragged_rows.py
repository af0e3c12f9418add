"""GPU parity of ragged rows on the vectorized kernel: persistent launches of many rows whose
length is not a whole number of 16-byte chunks, or whose row tensors start at addresses or
row strides that are only element-aligned. Those rows are addressed by byte: every chunk as a
16-byte access at element alignment through a buffer resource that ends with the row (the
partial last chunk moves its whole dwords), and the last element of an odd-length 16-bit row
by one 2-byte access. Every case is checked against the fp64 oracle (the same bars as the
aligned rows),
the plan is checked to be that path, and the bytes around every output row (row padding,
the elements before and after the tensors) are checked to be left as they were.

Cases cover every partial-chunk length of each dtype (fp32: 1-3 elements, 16-bit: 1-7),
rows of one chunk or less, every row-group width (1 to 16 waves), all five operations with
and without parameters, misaligned tensors with whole-chunk rows, odd row strides, and
outputs written over their inputs. (16-bit rows at odd 2-byte positions of the fused ops from
4 waves per row and of RMSNorm from 8 take the pair kernel instead, by measurement: those
shapes are left to the planner tests.)"""

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
BASE = {"ln": workloads.C1, "rms": workloads.C3, "fused_add_rms": workloads.C4_FP16, "fused_add_ln": workloads.FUSED_LN,
        "softmax": workloads.SOFTMAX}
TD = workloads.TORCH_DTYPES
SENTINEL = {torch.float32: 0x7FC0DEAD, torch.float16: 0x7E5A, torch.bfloat16: 0x7FDA}  # NaN payloads


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


def _bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


class Placed:
    """A [rows, N] tensor inside a larger buffer: element offset `off`, row stride `ld`; the
    rest of the buffer holds a sentinel so that stray writes show."""

    def __init__(self, rows, N, dtype, off, ld, src=None):
        self.buf = torch.empty(off + rows * ld + 16, dtype=dtype, device=DEV)
        _bits(self.buf).fill_(SENTINEL[dtype])
        self.view = self.buf[off:off + rows * ld].view(rows, ld)[:, :N]
        if src is not None:
            self.view.copy_(src.to(DEV))
        self.before = self.buf.clone()

    def untouched_outside(self):
        mask = torch.ones_like(self.buf, dtype=torch.bool)
        mask[self.view.storage_offset():self.view.storage_offset() + self.view.shape[0] * self.view.stride(0)].view(
            self.view.shape[0], self.view.stride(0))[:, :self.view.shape[1]] = False
        return torch.equal(_bits(self.buf)[mask], _bits(self.before)[mask])


def run_case(op, dtype, rows, N, *, seed, gamma=True, beta=True, off=None, ld=None, in_place=False):
    """One call through the binding with the given placement; returns the plan it took."""
    w = BASE[op].scaled(rows=rows, N=N, seed=seed, dtype=dtype, with_gamma=gamma, with_beta=beta)
    inp = workloads.make_inputs(w)
    ref = _oracle(w, inp)
    td = TD[dtype]
    off = off or {}
    ld = ld or {}
    names = ["x", "y"] + (["residual", "residual_out"] if op in ("fused_add_rms", "fused_add_ln") else [])
    pl = {}
    for k in names:
        src = inp.get(k) if k in ("x", "residual") else None
        pl[k] = Placed(rows, N, td, off.get(k, 0), ld.get(k, N), src)
    if in_place:
        pl["y"] = pl["x"]
        if "residual" in pl:
            pl["residual_out"] = pl["residual"]
    x = pl["x"].view
    g = inp.get("gamma", inp.get("weight"))
    g = None if g is None else g.to(DEV)
    b = inp["beta"].to(DEV) if "beta" in inp else None
    ptrs = {k: p.view.data_ptr() for k, p in pl.items()}
    if g is not None:
        ptrs["gamma"] = g.data_ptr()
    if b is not None:
        ptrs["beta"] = b.data_ptr()
    strides = {k: p.view.stride(0) for k, p in pl.items() if p.view.stride(0) != N}
    st, info = rn.plan(op, rows, N, td, ptrs=ptrs, strides=strides or None, eps=w.eps)
    assert st == 0, st
    out = {}
    if op == "ln":
        y, m, r = rn.ln_forward(x, g, b, w.eps, out=pl["y"].view, return_stats=True)
        out = {"y": y, "mean": m, "rstd": r}
    elif op == "rms":
        y, r = rn.rms_norm(x, g, w.eps, out=pl["y"].view, return_rstd=True)
        out = {"y": y, "rstd": r}
    elif op == "fused_add_rms":
        y, ro, r = rn.fused_add_rms_norm(x, pl["residual"].view, g, w.eps, out=pl["y"].view,
                                         residual_out=pl["residual_out"].view, return_rstd=True)
        out = {"y": y, "residual_out": ro, "rstd": r}
    elif op == "fused_add_ln":
        y, ro, m, r = rn.fused_add_layer_norm(x, pl["residual"].view, g, b, w.eps, out=pl["y"].view,
                                              residual_out=pl["residual_out"].view, return_stats=True)
        out = {"y": y, "residual_out": ro, "mean": m, "rstd": r}
    else:
        y, mx, sm = rn.softmax_forward(x, out=pl["y"].view, return_stats=True)
        out = {"y": y, "max": mx, "sum": sm}
    torch.cuda.synchronize()
    if op == "softmax":
        check_softmax_y(out["y"], ref["y"])
        check_equal_values(out["max"], ref["max"], "row_max")
        check_rel(out["sum"], ref["sum"], STAT_REL_TOL, "row_sum")
    else:
        check_y(out["y"], ref["y"], "y", op=op)
        check_rstd(out["rstd"], ref["rstd"])
        if "mean" in out:
            check_mean(out["mean"], ref["mean"], ref["rstd"], w.eps)
        if "residual_out" in out:
            check_bits_equal(out["residual_out"], ref["residual_out"], "residual_out")
    for k in ("y", "residual_out"):
        if k in pl:
            assert pl[k].untouched_outside(), f"{k}: bytes outside the rows were written"
    return info


# (op, dtype, rows, N, gamma, beta): every partial-chunk length, every row-group width
SHAPES = [
    ("ln", "bf16", 1024, 4095, True, True),      # 2 waves, 7 of 8 in the last chunk
    ("ln", "bf16", 600, 4093, True, False),      # 5 of 8, gamma only
    ("ln", "fp16", 1030, 1001, False, False),    # 1 wave x 2 chunks, 1 of 8, no parameters
    ("ln", "fp32", 300, 4095, True, True),       # 4 waves, 3 of 4
    ("ln", "fp32", 260, 16383, True, True),      # 16 waves, 3 of 4 (no fp32 copy, gamma in VGPRs)
    ("ln", "fp32", 2048, 3, True, True),         # rows shorter than a chunk: only a partial chunk
    ("ln", "fp32", 1100, 1022, False, True),     # 1 wave x 4 chunks, 2 of 4, beta only
    ("rms", "fp16", 1100, 2047, True, False),    # 1 wave x 4 chunks, 7 of 8
    ("rms", "fp32", 280, 8191, False, False),    # 8 waves, 3 of 4, no weight
    ("rms", "bf16", 280, 16382, False, False),   # 8 waves, 6 of 8 (rows at 4-byte positions)
    ("rms", "bf16", 1024, 9, True, False),       # one whole chunk and 1 element
    ("rms", "fp32", 520, 2049, True, False),     # 4 waves: 513 chunks of 1024 slots, 1 of 4
    ("fused_add_rms", "fp16", 520, 4094, True, False),   # 6 of 8
    ("fused_add_rms", "bf16", 1040, 1003, False, False),  # 1 wave, 3 of 8
    ("fused_add_ln", "bf16", 270, 8190, True, True),     # 4 waves, 6 of 8
    ("fused_add_ln", "fp32", 300, 3001, True, True),     # 4 waves, 1 of 4
    ("softmax", "fp32", 300, 4097, False, False),        # 8 waves: 1025 chunks of 2048 slots, 1 of 4
    ("softmax", "bf16", 300, 32767, False, False),       # 16 waves, 7 of 8
    ("softmax", "fp16", 1030, 444, False, False),        # 1 wave x 1 chunk, 4 of 8
]


@pytest.mark.parametrize("op,dtype,rows,N,gamma,beta", SHAPES,
                         ids=[f"{s[0]}-{s[1]}-{s[2]}x{s[3]}" for s in SHAPES])
def test_ragged_rows_against_the_oracle(op, dtype, rows, N, gamma, beta):
    info = run_case(op, dtype, rows, N, seed=1900 + N % 97, gamma=gamma, beta=beta)
    assert info["ragged"] and info["persistent"], info


@pytest.mark.parametrize("op,dtype,rows,N,off,ld", [
    ("ln", "bf16", 512, 4096, {"x": 1, "y": 3}, None),                  # whole chunks, misaligned tensors
    ("ln", "fp32", 256, 4096, {"x": 1}, {"y": 4099}),                    # misaligned x, padded odd y stride
    ("rms", "fp32", 1024, 1024, None, {"x": 1025, "y": 1027}),          # odd row strides
    ("rms", "fp16", 2048, 1000, {"x": 7, "y": 5}, {"x": 1001}),          # whole chunks per row, odd stride
    ("fused_add_rms", "bf16", 520, 4000, {"x": 1, "residual": 2, "y": 3, "residual_out": 5}, None),
    ("fused_add_ln", "fp16", 270, 8190, {"x": 2, "residual": 4}, {"y": 8194, "residual_out": 8192}),
    ("fused_add_ln", "fp32", 270, 4095, {"x": 3, "residual": 1}, {"y": 4099, "residual_out": 4097}),
    ("softmax", "fp32", 300, 8192, {"x": 2, "y": 1}, None),
])
def test_misaligned_tensors_and_strides(op, dtype, rows, N, off, ld):
    info = run_case(op, dtype, rows, N, seed=1950 + rows % 89, off=off, ld=ld)
    assert info["ragged"] and info["persistent"], info


@pytest.mark.parametrize("op,dtype,rows,N", [("ln", "bf16", 1024, 4095), ("fused_add_ln", "fp32", 300, 3001),
                                             ("fused_add_rms", "fp16", 520, 4094), ("softmax", "bf16", 1030, 1001)])
def test_ragged_rows_in_place(op, dtype, rows, N):
    # y over x (and residual_out over residual): each lane loads its chunks before it stores them
    info = run_case(op, dtype, rows, N, seed=1990 + rows % 7, off={"x": 1, "residual": 3}, in_place=True)
    assert info["ragged"], info


def test_few_ragged_rows_keep_the_element_kernels():
    # under 256 row blocks the launch is not persistent: the element / pair kernels
    for op, dtype, rows, N in (("ln", "bf16", 300, 4095), ("rms", "fp32", 200, 4095), ("softmax", "fp16", 1000, 999)):
        info = run_case(op, dtype, rows, N, seed=2000 + rows)
        assert info["variant"] == "element" and not info["ragged"], info


@pytest.mark.parametrize("dtype,rows,N,V,off,in_place", [
    ("fp32", 300, 50257, 16, None, False),   # vocabulary rows: 12565 chunks, the last 1 of 4
    ("bf16", 200, 40001, 8, None, False),    # 5001 chunks, the last 1 of 8 (an odd length)
    ("fp16", 64, 65535, 8, None, False),     # 8192 chunks, the last 7 of 8
    ("fp32", 7, 16385, 8, None, False),      # 4097 chunks, few rows
    ("fp32", 9, 65535, 16, None, False),     # 16384 chunks, the last 3 of 4
    ("fp32", 100, 50304, 16, {"x": 1, "y": 3}, False),  # whole chunks at element-aligned addresses
    ("bf16", 50, 50257, 8, {"x": 1}, True),  # in place, rows at odd 2-byte positions
])
def test_vocabulary_softmax_rows(dtype, rows, N, V, off, in_place):
    # softmax rows of more than 4096 chunks that are not whole chunks: byte-addressed rows on
    # one 16-wave workgroup each, grid per row
    info = run_case("softmax", dtype, rows, N, seed=2300 + N % 101, off=off, in_place=in_place)
    assert info["ragged"] and not info["persistent"], info
    assert (info["waves_per_row"], info["chunks_per_lane"]) == (16, V), info
