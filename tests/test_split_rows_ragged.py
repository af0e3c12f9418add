"""GPU parity of the one-pass split-row forward on byte-addressed rows: rows longer than one
workgroup holds whose length, row stride or tensor addresses are not whole 16-byte chunks. The
segments of such a row move through buffer resources that end with the segment (the last one
with the row): 16-byte accesses at element alignment, the row's partial last chunk by its
whole dwords and, for odd-length 16-bit rows, its last element by one 2-byte access. Checked
against the fp64 oracle, against the element-granular two-launch form (8192-element segments:
other segment sums, so within the same bars rather than bit for bit), with every record of a
row computed from memory by each of the row's workgroups (RN_FWD_WAIT_POLLS=0: the same bits,
which pins the partial chunk's handling in the path that computes another segment's record),
and with the bytes around every output row left as they were."""

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
LIB = rn._lib
OPS = {"ln": 0, "rms": 1, "fused_add_rms": 2, "fused_add_ln": 3, "softmax": 4}
DT = {"fp32": 0, "fp16": 1, "bf16": 2}
ESZ = {"fp32": 4, "fp16": 2, "bf16": 2}
AUTO, WIDE_ELEMENT = 0, 6


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def _forward(w, g, ws, variant=AUTO):
    o = {"y": torch.full_like(g["x"], float("nan")), "rstd": torch.full((w.rows,), float("nan"), device=DEV),
         "mean": torch.full((w.rows,), float("nan"), device=DEV)}
    if w.op in ("fused_add_rms", "fused_add_ln"):
        o["residual_out"] = torch.full_like(g["x"], float("nan"))
    if w.op in ("rms", "fused_add_rms"):
        o.pop("mean")
    st = LIB.rn_forward_ex(OPS[w.op], _p(g["x"]), _p(g.get("residual")), _p(g.get("gamma", g.get("weight"))),
                           _p(g.get("beta")), _p(o["y"]), _p(o.get("residual_out")), _p(o.get("mean")), _p(o["rstd"]),
                           w.rows, w.N, ctypes.c_float(w.eps), DT[w.dtype], None, variant, _p(ws),
                           ctypes.c_size_t(ws.numel()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, rn.STATUS.get(st, st)
    return o


def _oracle(w, inp):
    if w.op == "softmax":
        return oracle.softmax(inp["x"], threads=THREADS)
    if w.op == "ln":
        return oracle.layer_norm(inp["x"], inp.get("gamma"), inp.get("beta"), w.eps, threads=THREADS)
    if w.op == "rms":
        return oracle.rms_norm(inp["x"], inp.get("weight"), w.eps, threads=THREADS)
    if w.op == "fused_add_rms":
        return oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp.get("weight"), w.eps, threads=THREADS)
    return oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp.get("gamma"), inp.get("beta"), w.eps,
                                       threads=THREADS)


def _check(w, ref, o):
    if w.op == "softmax":
        check_softmax_y(o["y"], ref["y"])
        check_equal_values(o["mean"], ref["max"], "row_max")
        check_rel(o["rstd"], ref["sum"], STAT_REL_TOL, "row_sum")
        return
    check_y(o["y"], ref["y"], "y", op=w.op)
    check_rstd(o["rstd"], ref["rstd"])
    if "mean" in o:
        check_mean(o["mean"], ref["mean"], ref["rstd"], w.eps)
    if "residual_out" in o:
        check_bits_equal(o["residual_out"], ref["residual_out"], "residual_out")


CASES = [
    # (base workload, dtype, rows, N): the last segment ends with a chunk of N mod E elements.
    # 16-bit rows of odd length take this path only as a single row (several such rows sit at
    # odd 2-byte positions, which the planner gives to the element-granular two launches):
    # those cases move the row's last element by the 2-byte access.
    (workloads.C2, "fp32", 40, 65537),        # 1 of 4; the last segment holds only that chunk
    (workloads.C2, "fp32", 40, 65538),        # 2 of 4
    (workloads.C1, "fp32", 40, 65539),        # 3 of 4
    (workloads.C5, "bf16", 1, 65537),         # 1 of 8 (the 2-byte access alone)
    (workloads.C5, "bf16", 32, 65538),        # 2 of 8
    (workloads.C5, "bf16", 1, 65539),         # 3 of 8
    (workloads.C5, "fp16", 32, 65540),        # 4 of 8
    (workloads.C5, "bf16", 1, 65541),         # 5 of 8
    (workloads.C5, "fp16", 32, 65542),        # 6 of 8
    (workloads.C5, "bf16", 1, 65543),         # 7 of 8
    (workloads.C5, "bf16", 24, 20002),        # two segments
    (workloads.C3, "fp16", 32, 50002),
    (workloads.C3, "fp16", 1, 50001),
    (workloads.C4_FP16, "fp16", 24, 70002),
    (workloads.C4_FP16, "fp16", 1, 70001),
    (workloads.C4_BF16, "bf16", 24, 65538),
    (workloads.FUSED_LN, "bf16", 1, 50003),
    (workloads.FUSED_LN, "bf16", 24, 50006),
    (workloads.FUSED_LN.scaled(dtype="fp32"), "fp32", 16, 40001),
    (workloads.SOFTMAX, "fp32", 16, 100003),
    (workloads.SOFTMAX, "bf16", 16, 70002),
    (workloads.SOFTMAX, "bf16", 1, 70001),
]


@pytest.mark.parametrize("base,dtype,rows,N", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_byte_addressed_one_pass(base, dtype, rows, N, monkeypatch):
    w = base.scaled(rows=rows, N=N, seed=1700 + N % 101, dtype=dtype)
    inp = workloads.make_inputs(w)
    ref = _oracle(w, inp)
    g = {k: v.to(DEV) for k, v in inp.items()}
    td = g["x"].dtype
    need = rn.forward_workspace_bytes(w.op, rows, N, td)
    st, info = rn.plan(w.op, rows, N, td, workspace_bytes=need)
    assert st == 0 and info["variant"] == "wide" and info["ragged"], info
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    monkeypatch.delenv("RN_FWD_WAIT_POLLS", raising=False)
    one = _forward(w, g, ws)
    _check(w, ref, one)
    # every record computed from memory by each workgroup of its row: the same bits
    monkeypatch.setenv("RN_FWD_WAIT_POLLS", "0")
    local = _forward(w, g, ws)
    computed = int(ws[4:8].view(torch.int32).item())
    monkeypatch.delenv("RN_FWD_WAIT_POLLS")
    S = -(-(-(-N * ESZ[dtype] // 16)) // 2048)
    assert computed == rows * S * S
    for k in one:
        assert torch.equal(_bits(one[k]), _bits(local[k])), k
    # the element-granular two launches meet the oracle as well
    _check(w, ref, _forward(w, g, ws, WIDE_ELEMENT))


def _placed(rows, N, dtype, off, ld, src=None):
    buf = torch.full((off + rows * ld + 64,), float("nan"), dtype=dtype, device=DEV)
    view = buf[off:off + rows * ld].view(rows, ld)[:, :N]
    if src is not None:
        view.copy_(src.to(DEV))
    return buf, view


@pytest.mark.parametrize("op,dtype,rows,N,off,ld", [
    ("ln", "bf16", 16, 65536, {"x": 2, "y": 6}, {}),                     # whole chunks, misaligned tensors
    ("ln", "fp32", 12, 50000, {"x": 1}, {"y": 50003}),                  # padded odd stride
    ("ln", "fp32", 12, 50001, {"x": 3, "y": 2}, {"x": 50005}),
    ("rms", "fp16", 16, 40002, {"x": 2, "y": 4}, {"x": 40004}),
    ("fused_add_rms", "bf16", 12, 65536, {"x": 2, "residual": 4, "y": 6, "residual_out": 10}, {}),
    ("fused_add_ln", "fp16", 12, 33334, {"x": 2, "residual": 6}, {"y": 33338, "residual_out": 33336}),
    ("softmax", "fp32", 8, 70000, {"x": 2, "y": 1}, {}),
])
def test_byte_addressed_one_pass_placement(op, dtype, rows, N, off, ld):
    base = {"ln": workloads.C1, "rms": workloads.C3, "fused_add_rms": workloads.C4_FP16,
            "fused_add_ln": workloads.FUSED_LN, "softmax": workloads.SOFTMAX}[op]
    w = base.scaled(rows=rows, N=N, seed=1760 + rows, dtype=dtype)
    inp = workloads.make_inputs(w)
    ref = _oracle(w, inp)
    td = workloads.TORCH_DTYPES[dtype]
    names = ["x", "y"] + (["residual", "residual_out"] if op.startswith("fused") else [])
    bufs, views = {}, {}
    for k in names:
        bufs[k], views[k] = _placed(rows, N, td, off.get(k, 0), ld.get(k, N), inp.get(k))
    before = {k: bufs[k].clone() for k in ("y", "residual_out") if k in bufs}
    g = inp.get("gamma", inp.get("weight"))
    g = None if g is None else g.to(DEV)
    b = inp["beta"].to(DEV) if "beta" in inp else None
    ptrs = {k: v.data_ptr() for k, v in views.items()}
    strides = {k: v.stride(0) for k, v in views.items() if v.stride(0) != N}
    st, info = rn.plan(op, rows, N, td, ptrs=ptrs, strides=strides or None,
                       workspace_bytes=rn.forward_workspace_bytes(op, rows, N, td))
    assert st == 0 and info["variant"] == "wide" and info["ragged"], info
    x = views["x"]
    if op == "ln":
        y, m, r = rn.ln_forward(x, g, b, w.eps, out=views["y"], return_stats=True)
        o = {"y": y, "mean": m, "rstd": r}
    elif op == "rms":
        y, r = rn.rms_norm(x, g, w.eps, out=views["y"], return_rstd=True)
        o = {"y": y, "rstd": r}
    elif op == "fused_add_rms":
        y, ro, r = rn.fused_add_rms_norm(x, views["residual"], g, w.eps, out=views["y"],
                                         residual_out=views["residual_out"], return_rstd=True)
        o = {"y": y, "residual_out": ro, "rstd": r}
    elif op == "fused_add_ln":
        y, ro, m, r = rn.fused_add_layer_norm(x, views["residual"], g, b, w.eps, out=views["y"],
                                              residual_out=views["residual_out"], return_stats=True)
        o = {"y": y, "residual_out": ro, "mean": m, "rstd": r}
    else:
        y, mx, sm = rn.softmax_forward(x, out=views["y"], return_stats=True)
        o = {"y": y, "mean": mx, "rstd": sm}
    torch.cuda.synchronize()
    _check(w, ref, o)
    for k, b0 in before.items():  # nothing written outside the output rows
        mask = torch.ones_like(b0, dtype=torch.bool)
        v = views[k]
        mask[v.storage_offset():v.storage_offset() + rows * v.stride(0)].view(rows, v.stride(0))[:, :N] = False
        assert torch.equal(_bits(bufs[k])[mask], _bits(b0)[mask]), k


@pytest.mark.parametrize("op,dtype,rows,N", [("ln", "bf16", 24, 65539), ("fused_add_rms", "fp16", 16, 50001),
                                             ("softmax", "bf16", 8, 70001)])
def test_odd_position_16bit_rows_take_element_segments(op, dtype, rows, N):
    # several 16-bit rows of odd length sit at odd 2-byte positions: the element-granular two
    # launches (measured faster there than 16-byte accesses at those positions)
    base = {"ln": workloads.C5, "fused_add_rms": workloads.C4_FP16, "softmax": workloads.SOFTMAX}[op]
    w = base.scaled(rows=rows, N=N, seed=1790 + rows, dtype=dtype)
    inp = workloads.make_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    need = rn.forward_workspace_bytes(w.op, rows, N, g["x"].dtype)
    st, info = rn.plan(w.op, rows, N, g["x"].dtype, workspace_bytes=need)
    assert st == 0 and info["variant"] == "wide_element" and not info["ragged"], info
    _check(w, _oracle(w, inp), _forward(w, g, torch.empty(need, dtype=torch.uint8, device=DEV)))
