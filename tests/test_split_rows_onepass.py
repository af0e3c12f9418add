"""GPU parity of the one-pass split-row forward (rows of whole 16-byte chunks longer than one
workgroup holds): x is read once, the segments of a row exchange their statistics records
through the workspace. Checked bit for bit against the two-launch form (the same records,
combined in the same order; chosen by giving a workspace too small for the one-pass layout),
with every record computed from memory by every workgroup of its row (RN_FWD_WAIT_POLLS=0), and
against the fp64 oracle. Calls go through rn_forward_ex with device pointers."""

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
WIDE = 5  # RN_VARIANT_WIDE
ESZ = {"fp32": 4, "fp16": 2, "bf16": 2}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _two_pass_bytes(rows, N):
    return rows * (-(-N // 8192)) * 16


def _forward(w, g, ws):
    o = {"y": torch.full_like(g["x"], float("nan")), "rstd": torch.full((w.rows,), float("nan"), device=DEV),
         "mean": torch.full((w.rows,), float("nan"), device=DEV)}
    if w.op in ("fused_add_rms", "fused_add_ln"):
        o["residual_out"] = torch.full_like(g["x"], float("nan"))
    if w.op in ("rms", "fused_add_rms"):
        o.pop("mean")
    st = LIB.rn_forward_ex(OPS[w.op], _p(g["x"]), _p(g.get("residual")), _p(g.get("gamma", g.get("weight"))),
                           _p(g.get("beta")), _p(o["y"]), _p(o.get("residual_out")), _p(o.get("mean")), _p(o["rstd"]),
                           w.rows, w.N, ctypes.c_float(w.eps), DT[w.dtype], None, WIDE, _p(ws),
                           ctypes.c_size_t(ws.numel()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, rn.STATUS.get(st, st)
    return o


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _oracle_check(w, inp, o):
    if w.op == "softmax":
        ref = oracle.softmax(inp["x"], threads=THREADS)
        check_softmax_y(o["y"], ref["y"])
        check_equal_values(o["mean"], ref["max"], "row_max")
        check_rel(o["rstd"], ref["sum"], STAT_REL_TOL, "row_sum")
        return
    if w.op == "ln":
        ref = oracle.layer_norm(inp["x"], inp.get("gamma"), inp.get("beta"), w.eps, threads=THREADS)
    elif w.op == "rms":
        ref = oracle.rms_norm(inp["x"], inp.get("weight"), w.eps, threads=THREADS)
    elif w.op == "fused_add_rms":
        ref = oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp.get("weight"), w.eps, threads=THREADS)
    else:
        ref = oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp.get("gamma"), inp.get("beta"), w.eps,
                                          threads=THREADS)
    check_y(o["y"], ref["y"], "y", op=w.op)
    check_rstd(o["rstd"], ref["rstd"])
    if "mean" in o:
        check_mean(o["mean"], ref["mean"], ref["rstd"], w.eps)
    if "residual_out" in o:
        check_bits_equal(o["residual_out"], ref["residual_out"], "residual_out")


CASES = [
    # (base workload, dtype, rows, N): segments of 32 KiB; S = 8, 8, 3 (last partial), 4, 4, 4 (partial), 13 (partial)
    (workloads.C2, "fp32", 64, 65536),
    (workloads.C5, "bf16", 48, 131072),
    (workloads.C5, "fp16", 40, 40000),
    (workloads.C3, "fp16", 32, 65536),
    (workloads.C4_FP16, "fp16", 24, 65536),
    (workloads.FUSED_LN, "bf16", 24, 50000),
    (workloads.SOFTMAX, "fp32", 16, 100000),
    (workloads.SOFTMAX, "bf16", 16, 70000),
]


@pytest.mark.parametrize("base,dtype,rows,N", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_one_pass_matches_two_launches_and_oracle(base, dtype, rows, N, monkeypatch):
    w = base.scaled(rows=rows, N=N, seed=1600 + rows, dtype=dtype)
    inp = workloads.make_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    need = rn.forward_workspace_bytes(w.op, rows, N, g["x"].dtype)
    assert need > _two_pass_bytes(rows, N)
    monkeypatch.delenv("RN_FWD_WAIT_POLLS", raising=False)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    one = _forward(w, g, ws)
    assert int(ws[4:8].view(torch.int32).item()) >= 0  # the header was written (cleared) by the call
    two = _forward(w, g, torch.empty(_two_pass_bytes(rows, N), dtype=torch.uint8, device=DEV))
    for k in one:
        assert torch.equal(_bits(one[k]), _bits(two[k])), k
    # every record of a row computed by each of the row's workgroups from memory: the same
    # bits again
    monkeypatch.setenv("RN_FWD_WAIT_POLLS", "0")
    local = _forward(w, g, ws)
    computed = int(ws[4:8].view(torch.int32).item())
    monkeypatch.delenv("RN_FWD_WAIT_POLLS")
    S = -(-(N * ESZ[dtype]) // 32768)
    assert computed == rows * S * S
    for k in one:
        assert torch.equal(_bits(one[k]), _bits(local[k])), k
    _oracle_check(w, inp, one)


@pytest.mark.parametrize("base,dtype,rows,N", [
    (workloads.C2, "fp32", 333, 65536),        # blocks of 4 rows, then 65 rows in single-row tickets
    (workloads.FUSED_LN, "bf16", 320, 65536),  # 4 segments; blocks of several rows and a tail
], ids=lambda v: getattr(v, "name", str(v)))
def test_one_pass_blocks_and_tail_tickets(base, dtype, rows, N):
    # enough rows that blocks hold several rows (about rows / 4 blocks against the resident
    # grid's res / S) and the last round goes in single-row tickets
    w = base.scaled(rows=rows, N=N, seed=1660 + rows, dtype=dtype)
    inp = workloads.make_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    need = rn.forward_workspace_bytes(w.op, rows, N, g["x"].dtype)
    one = _forward(w, g, torch.empty(need, dtype=torch.uint8, device=DEV))
    two = _forward(w, g, torch.empty(_two_pass_bytes(rows, N), dtype=torch.uint8, device=DEV))
    for k in one:
        assert torch.equal(_bits(one[k]), _bits(two[k])), k
    _oracle_check(w, inp, one)


def test_in_place_split_rows_take_two_launches(monkeypatch):
    # In place (y over x; residual_out over the residual and y over x) a waiting workgroup
    # could compute another segment's record from data its owner has already overwritten,
    # so such calls take the two launches: with every record forced to be computed locally
    # the in-place results still meet the oracle and equal the out-of-place ones bit for bit.
    monkeypatch.setenv("RN_FWD_WAIT_POLLS", "0")
    w = workloads.C2.scaled(rows=32, N=65536, seed=1651)
    inp = workloads.make_inputs(w)
    ref = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], w.eps, threads=THREADS)
    g = {k: v.to(DEV) for k, v in inp.items()}
    y = rn.ln_forward(g["x"], g["gamma"], g["beta"], w.eps)
    x = g["x"].clone()
    rn.ln_forward(x, g["gamma"], g["beta"], w.eps, out=x)
    torch.cuda.synchronize()
    check_y(x, ref["y"], op="ln")
    assert torch.equal(_bits(x), _bits(y))
    w = workloads.C4_FP16.scaled(rows=16, N=65536, seed=1653)
    inp = workloads.make_inputs(w)
    ref = oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp["weight"], w.eps, threads=THREADS)
    g = {k: v.to(DEV) for k, v in inp.items()}
    x, r = g["x"].clone(), g["residual"].clone()
    ws = torch.empty(rn.forward_workspace_bytes("fused_add_rms", 16, 65536, torch.float16), dtype=torch.uint8,
                     device=DEV)
    st = LIB.rn_forward_ex(OPS["fused_add_rms"], _p(x), _p(r), _p(g["weight"]), None, _p(x), _p(r), None, None, 16,
                           65536, ctypes.c_float(w.eps), DT["fp16"], None, WIDE, _p(ws), ctypes.c_size_t(ws.numel()),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    check_y(x, ref["y"], op="fused_add_rms")
    check_bits_equal(r, ref["residual_out"], "residual_out in place")


def test_many_segments_take_two_launches():
    # rows of more than 256 segments (here 257 x 8192 fp32 elements) take the two launches
    w = workloads.C2.scaled(rows=3, N=257 * 8192, seed=1652)
    inp = workloads.make_inputs(w)
    ref = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], w.eps, threads=THREADS)
    y, mean, rstd = rn.ln_forward(inp["x"].to(DEV), inp["gamma"].to(DEV), inp["beta"].to(DEV), w.eps,
                                  return_stats=True)
    torch.cuda.synchronize()
    check_y(y, ref["y"], op="ln")
    check_mean(mean, ref["mean"], ref["rstd"], w.eps)
    check_rstd(rstd, ref["rstd"])


@pytest.mark.parametrize("op,dtype,N,variants", [("softmax", "bf16", 32768, ("wide_element",)),
                                                  ("rms", "fp16", 32768, ("wide_element",)),
                                                  ("ln", "bf16", 32768, ("wide_element",)),
                                                  ("rms", "fp16", 65536, ("wide", "wide_element"))])
def test_forced_split_rows_through_the_binding(op, dtype, N, variants):
    # rows of whole chunks that the automatic plan holds in one workgroup (64 and 128 KiB): a
    # forced split-row variant through the Python binding gets its workspace from the binding
    # (16-byte segments only for rows of more than 4096 chunks)
    base = {"softmax": workloads.SOFTMAX, "rms": workloads.C3, "ln": workloads.C5}[op]
    w = base.scaled(rows=37, N=N, seed=2250 + N % 7, dtype=dtype)
    inp = workloads.make_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    for variant in variants:
        if op == "softmax":
            y, mx, sm = rn.softmax_forward(g["x"], return_stats=True, variant=variant)
            o = {"y": y, "mean": mx, "rstd": sm}
        elif op == "rms":
            y, r = rn.rms_norm(g["x"], g.get("weight"), w.eps, return_rstd=True, variant=variant)
            o = {"y": y, "rstd": r}
        else:
            y, m, r = rn.ln_forward(g["x"], g.get("gamma"), g.get("beta"), w.eps, return_stats=True, variant=variant)
            o = {"y": y, "mean": m, "rstd": r}
        torch.cuda.synchronize()
        _oracle_check(w, inp, o)
