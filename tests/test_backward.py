"""GPU parity of the backward passes (LayerNorm, RMSNorm) against the fp64 oracle.

The forward statistics fed to both sides are the oracle's fp64 mean / rstd rounded to fp32
(the dtype the forward stores), so both evaluate the same formula at the same point. Tolerances
are derived in tests/_compare.py (check_dx, check_colsum); the column-sum depth comes from the
launch plan: rows per lane, the row groups of a workgroup, and the P partial rows.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import row_wise_normalization_fp32_amd as rn
import workloads
from _compare import check_colsum, check_dx

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def _stats(w, inp):
    if w.op == "ln_bwd":
        f = oracle.layer_norm(inp["x"], None, None, w.eps, threads=min(16, os.cpu_count() or 1), want_y=False)
        return f["mean"].astype(np.float32), f["rstd"].astype(np.float32)
    f = oracle.rms_norm(inp["x"], None, w.eps, threads=min(16, os.cpu_count() or 1), want_y=False)
    return None, f["rstd"].astype(np.float32)


def _scales(w, inp, mean, rstd, gamma):
    """Row scales for dx and absolute column sums for dgamma / dbeta (tolerance scales,
    from the inputs)."""
    x = inp["x"].double().numpy()
    dy = inp["dy"].double().numpy()
    r = rstd.astype(np.float64)[:, None]
    xh = (x - mean.astype(np.float64)[:, None]) * r if mean is not None else x * r
    g = dy * (gamma.double().numpy()[None, :] if gamma is not None else 1.0)
    row = r[:, 0] * np.abs(g).max(axis=1) * np.maximum(1.0, np.abs(xh).max(axis=1)) ** 2
    return row, np.abs(dy * xh).sum(axis=0), np.abs(dy).sum(axis=0)


def _depth(op, rows, N, dtype):
    st, info = rn.plan_backward(op, rows, N, TD[dtype], ptrs={"workspace": 1 << 46})
    assert st == 0, st
    # the launch uses P = min(grid, CUs x resident workgroups per CU) partial rows: at least
    # one workgroup per CU (rows per lane), at most the plan's grid (partial rows per lane
    # of the column kernel). Split rows: P = min(grid, resident workgroups / S) per segment,
    # at least one.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rpb = info["rows_per_block"]
    if info["variant"] == "wide":
        S = -(-N // 8192)
        per_lane = -(-rows // max(1, min(info["grid_blocks"], cus // S)))
    else:
        per_lane = -(-rows // (min(info["grid_blocks"], cus) * rpb))
    return per_lane + rpb + info["grid_blocks"] / 16 + 16


def run_case(w, with_gamma=True, in_place=False, params=True):
    inp = workloads.make_inputs(w)
    gamma = inp.get("gamma" if w.op == "ln_bwd" else "weight") if with_gamma else None
    mean, rstd = _stats(w, inp)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    g_dev = gamma.to(DEV) if gamma is not None else None
    rstd_d = torch.from_numpy(rstd).to(DEV)
    if w.op == "ln_bwd":
        ref = oracle.layer_norm_backward(inp["dy"], inp["x"], gamma, mean=mean, rstd=rstd, eps=w.eps)
        mean_d = torch.from_numpy(mean).to(DEV)
        dyv = dev["dy"].clone()
        dx, dg, db = rn.ln_backward(dyv, dev["x"], mean_d, rstd_d, g_dev, dx=dyv if in_place else None,
                                    want_dgamma=params, want_dbeta=params)
    else:
        ref = oracle.rms_norm_backward(inp["dy"], inp["x"], gamma, rstd=rstd, eps=w.eps)
        dyv = dev["dy"].clone()
        dx, dg = rn.rms_norm_backward(dyv, dev["x"], rstd_d, g_dev, dx=dyv if in_place else None,
                                      want_dweight=params)
        db = None
    torch.cuda.synchronize()
    row, a_g, a_b = _scales(w, inp, mean, rstd, gamma)
    check_dx(dx, ref["dx"], row)
    if not params:
        assert dg is None and db is None
        return
    depth = _depth("ln" if w.op == "ln_bwd" else "rms", w.rows, w.N, w.dtype)
    check_colsum(dg, ref["dgamma" if w.op == "ln_bwd" else "dweight"], a_g, depth, "dgamma")
    if db is not None:
        check_colsum(db, ref["dbeta"], a_b, depth, "dbeta")


@pytest.mark.parametrize("w", [workloads.LN_BWD, workloads.RMS_BWD], ids=lambda w: w.name)
def test_backward_full_size(w):
    run_case(w)


SHAPES = [(37, 1000), (5, 4096), (9, 2056), (3, 8), (64, 1024), (33, 333), (6, 16384), (4, 12289), (300, 64)]


@pytest.mark.parametrize("op", ["ln_bwd", "rms_bwd"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_backward_shapes(op, dtype):
    base = workloads.LN_BWD if op == "ln_bwd" else workloads.RMS_BWD
    for rows, N in SHAPES:
        run_case(base.scaled(rows=rows, N=N, seed=1200 + N, dtype=dtype))


# Rows longer than 16384 elements: split into 8192-element segments (16-byte groups when
# N * s is a multiple of 16, else element by element), ragged last segments included.
LONG = [("ln_bwd", "bf16", 24, 32768), ("ln_bwd", "fp32", 12, 50001), ("ln_bwd", "fp16", 40, 16392),
        ("rms_bwd", "fp16", 16, 65536), ("rms_bwd", "bf16", 8, 20001), ("rms_bwd", "fp32", 10, 24580)]


@pytest.mark.parametrize("op,dtype,rows,N", LONG, ids=lambda v: str(v))
def test_backward_split_rows(op, dtype, rows, N):
    base = workloads.LN_BWD if op == "ln_bwd" else workloads.RMS_BWD
    w = base.scaled(rows=rows, N=N, seed=1300 + N, dtype=dtype)
    assert rn.plan_backward("ln" if op == "ln_bwd" else "rms", rows, N, TD[dtype],
                            ptrs={"workspace": 1 << 46})[1]["variant"] == "wide"
    run_case(w)


@pytest.mark.parametrize("op", ["ln_bwd", "rms_bwd"])
def test_backward_split_rows_variants(op):
    base = workloads.LN_BWD if op == "ln_bwd" else workloads.RMS_BWD
    run_case(base.scaled(rows=6, N=40960, seed=1320, dtype="bf16"), with_gamma=False)
    run_case(base.scaled(rows=6, N=40960, seed=1321, dtype="bf16"), in_place=True)
    run_case(base.scaled(rows=5, N=33333, seed=1322, dtype="fp32"), in_place=True, params=False)  # dx only
    run_case(base.scaled(rows=7, N=32768, seed=1323, dtype="fp16"), params=False)
    # more rows than workgroups per segment: each workgroup loops over rows
    run_case(base.scaled(rows=600, N=16392, seed=1324, dtype="bf16"))


# Rows of more than 64 segments: each lane of the waiting wave adds several records of the
# row. Rows of so many segments that the device keeps fewer than 2 S one-pass workgroups
# resident (S > 128 for the one-workgroup-per-CU instances: fp32, and rows that are not whole
# 16-byte groups) take the statistics + dx launches instead.
MANY_SEGMENTS = [("ln_bwd", "bf16", 3, 1100000), ("rms_bwd", "fp32", 2, 1100000), ("ln_bwd", "fp16", 2, 2200005)]


@pytest.mark.parametrize("op,dtype,rows,N", MANY_SEGMENTS, ids=lambda v: str(v))
def test_backward_split_rows_many_segments(op, dtype, rows, N):
    base = workloads.LN_BWD if op == "ln_bwd" else workloads.RMS_BWD
    run_case(base.scaled(rows=rows, N=N, seed=1350 + rows, dtype=dtype))


@pytest.mark.parametrize("dtype,N", [("bf16", 40960), ("fp32", 40001)])
def test_backward_split_rows_one_and_two_pass_agree(dtype, N):
    # a workspace that is only 4-byte aligned takes the three-launch form: both forms combine
    # the same segment sums in the same order, so dx has the same bits; the parameter
    # gradients (grouped into other partial rows) both meet the oracle's bound
    rows = 48
    w = workloads.LN_BWD.scaled(rows=rows, N=N, seed=1360, dtype=dtype)
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    ref = oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"], mean=mean, rstd=rstd, eps=w.eps)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    m, r = torch.from_numpy(mean).to(DEV), torch.from_numpy(rstd).to(DEV)
    need = rn.backward_workspace_bytes("ln", rows, N)
    ws = torch.empty(need + 16, dtype=torch.uint8, device=DEV)
    one = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], workspace=ws[:need])
    two = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], workspace=ws[4:need + 4])
    torch.cuda.synchronize()
    assert torch.equal(one[0].view(torch.uint8), two[0].view(torch.uint8))
    _, a_g, a_b = _scales(w, inp, mean, rstd, inp["gamma"])
    depth = _depth("ln", rows, N, dtype)
    for outs in (one, two):
        check_colsum(outs[1], ref["dgamma"], a_g, depth, "dgamma")
        check_colsum(outs[2], ref["dbeta"], a_b, depth, "dbeta")


def test_backward_split_rows_workspace_contents_do_not_matter():
    # the one-pass launch takes tickets from a counter and polls records in the workspace;
    # both are cleared by the call itself: a workspace full of ones (every record "ready")
    # gives the same bits as a fresh one, and the count of records computed by waiting
    # workgroups (the second 32-bit word of the 256-byte header in front of the rows x S
    # 16-byte records) starts from zero
    rows, N = 256, 65536
    w = workloads.LN_BWD.scaled(rows=rows, N=N, seed=1341, dtype="bf16")
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    m, r = torch.from_numpy(mean).to(DEV), torch.from_numpy(rstd).to(DEV)
    need = rn.backward_workspace_bytes("ln", rows, N)
    header = need - (256 + rows * (N // 8192) * 16)
    ref = [o.clone() for o in rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"])]
    for fill in (0xFF, 0x00):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        outs = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        assert 0 <= int(ws[header + 4:header + 8].view(torch.int32).item()) <= rows * (N // 8192)


def test_backward_split_rows_in_place_take_two_launches(monkeypatch):
    # dx over dy or over x: a waiting workgroup could compute another segment's sums from
    # data its owner has already overwritten, so in-place split rows take the three
    # launches; with every record forced to be computed locally the results keep their bits
    monkeypatch.setenv("RN_BWD_WAIT_POLLS", "0")
    w = workloads.LN_BWD.scaled(rows=48, N=65536, seed=1390, dtype="bf16")
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    m, r = torch.from_numpy(mean).to(DEV), torch.from_numpy(rstd).to(DEV)
    ref = [o.clone() for o in rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"])]
    for over in ("dy", "x"):
        t = {k: dev[k].clone() for k in ("dy", "x")}
        out = rn.ln_backward(t["dy"], t["x"], m, r, dev["gamma"], dx=t[over])
        torch.cuda.synchronize()
        assert out[0].data_ptr() == t[over].data_ptr()
        check_dx(out[0], oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"], mean=mean, rstd=rstd,
                                                     eps=w.eps)["dx"], _scales(w, inp, mean, rstd, inp["gamma"])[0])
        assert torch.equal(out[0].view(torch.uint8), ref[0].view(torch.uint8))


@pytest.mark.parametrize("op,dtype,rows,N,gamma", [("ln", "bf16", 96, 65536, True), ("ln", "fp32", 40, 40001, True),
                                                   ("rms", "fp16", 64, 32768, True), ("ln", "fp16", 48, 24576, False),
                                                   ("rms", "bf16", 33, 16392, False)])
def test_backward_split_rows_records_computed_by_the_waiting_workgroup(monkeypatch, op, dtype, rows, N, gamma):
    # RN_BWD_WAIT_POLLS=0: a workgroup polls each record of a row once and computes every
    # record not yet published itself, from that segment's x, dy and gamma. It uses the
    # lanes and the order of the segment's own workgroup, so dx, dgamma and dbeta have the
    # same bits as with the normal wait; the diagnostic count in the workspace header shows
    # that records were computed that way. Every kernel still ends normally: nothing waits
    # for a workgroup that is not running.
    base = workloads.LN_BWD if op == "ln" else workloads.RMS_BWD
    w = base.scaled(rows=rows, N=N, seed=1370 + rows, dtype=dtype, with_gamma=gamma)
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    r = torch.from_numpy(rstd).to(DEV)
    g = dev.get("gamma", dev.get("weight"))
    need = rn.backward_workspace_bytes(op, rows, N)
    S = -(-N // 8192)
    header = need - (256 + rows * S * 16)

    def call(ws):
        if op == "ln":
            out = rn.ln_backward(dev["dy"], dev["x"], torch.from_numpy(mean).to(DEV), r, g, workspace=ws)
        else:
            out = rn.rms_norm_backward(dev["dy"], dev["x"], r, g, workspace=ws)
        torch.cuda.synchronize()
        return [o.clone() for o in out if o is not None]

    monkeypatch.delenv("RN_BWD_WAIT_POLLS", raising=False)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    normal = call(ws)
    monkeypatch.setenv("RN_BWD_WAIT_POLLS", "0")
    local = call(ws)
    computed = int(ws[header + 4:header + 8].view(torch.int32).item())
    monkeypatch.delenv("RN_BWD_WAIT_POLLS")
    assert 0 < computed <= rows * S * (S - 1)  # each workgroup of a row may compute the others
    for a, b in zip(normal, local):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    # and against the oracle
    if op == "ln":
        ref = oracle.layer_norm_backward(inp["dy"], inp["x"], inp.get("gamma"), mean=mean, rstd=rstd, eps=w.eps)
    else:
        ref = oracle.rms_norm_backward(inp["dy"], inp["x"], inp.get("weight"), rstd=rstd, eps=w.eps)
    gam = inp.get("gamma", inp.get("weight"))
    s_r, a_g, a_b = _scales(w, inp, mean, rstd, gam)
    check_dx(local[0], ref["dx"], s_r)


def test_backward_split_rows_deterministic_and_param_only():
    w = workloads.LN_BWD.scaled(rows=64, N=24576, seed=1330, dtype="bf16")
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    m, r = torch.from_numpy(mean).to(DEV), torch.from_numpy(rstd).to(DEV)
    first = [o.clone() for o in rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"])]
    for _ in range(3):
        outs = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"])
        torch.cuda.synchronize()
        for a, b in zip(first, outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    # parameter gradients alone give the same bits
    _, dg, db = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], want_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dg.view(torch.uint8), first[1].view(torch.uint8))
    assert torch.equal(db.view(torch.uint8), first[2].view(torch.uint8))


@pytest.mark.parametrize("op", ["ln_bwd", "rms_bwd"])
def test_backward_without_gamma_and_in_place(op):
    base = workloads.LN_BWD if op == "ln_bwd" else workloads.RMS_BWD
    run_case(base.scaled(rows=64, N=4096, seed=1210), with_gamma=False)
    run_case(base.scaled(rows=64, N=4096, seed=1211), in_place=True)
    run_case(base.scaled(rows=64, N=1001, seed=1212), in_place=True)  # element kernel


def test_backward_offset_rows_and_many_rows():
    # rows far from zero (the cancellation case of the forward) and more rows than the
    # partial-row cap (several rows per lane)
    run_case(workloads.LN_BWD.scaled(rows=256, N=4096, seed=1220, dtype="fp32", x_dist="row_offset",
                                     row_offset=1000.0))
    run_case(workloads.LN_BWD.scaled(rows=16384, N=1024, seed=1221, dtype="bf16"))
    run_case(workloads.RMS_BWD.scaled(rows=16384, N=512, seed=1222, dtype="fp16"))


def test_backward_partial_outputs_and_zero_rows():
    w = workloads.LN_BWD.scaled(rows=32, N=2048, seed=1230)
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    ref = oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"], mean=mean, rstd=rstd, eps=w.eps)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    m, r = torch.from_numpy(mean).to(DEV), torch.from_numpy(rstd).to(DEV)
    dx, dg, db = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], want_dgamma=False, want_dbeta=False)
    assert dg is None and db is None
    row, a_g, a_b = _scales(w, inp, mean, rstd, inp["gamma"])
    torch.cuda.synchronize()
    check_dx(dx, ref["dx"], row)
    dx, dg, db = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], want_dx=False)
    torch.cuda.synchronize()
    assert dx is None
    depth = _depth("ln", 32, 2048, "bf16")
    check_colsum(dg, ref["dgamma"], a_g, depth, "dgamma")
    check_colsum(db, ref["dbeta"], a_b, depth, "dbeta")
    # one parameter gradient alone (the column pass runs one workgroup column per parameter)
    _, dg, db = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], want_dx=False, want_dgamma=False)
    torch.cuda.synchronize()
    assert dg is None
    check_colsum(db, ref["dbeta"], a_b, depth, "dbeta")
    _, dg, db = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"], want_dx=False, want_dbeta=False)
    torch.cuda.synchronize()
    assert db is None
    check_colsum(dg, ref["dgamma"], a_g, depth, "dgamma")
    # rows == 0: the parameter gradients are sums over no rows
    e = torch.empty(0, 64, device=DEV, dtype=torch.bfloat16)
    z = torch.empty(0, device=DEV)
    dx, dg, db = rn.ln_backward(e, e, z, z, torch.ones(64, device=DEV, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert dx.shape == (0, 64) and torch.equal(dg, torch.zeros_like(dg)) and torch.equal(db, torch.zeros_like(db))


def test_backward_is_deterministic():
    w = workloads.LN_BWD.scaled(rows=2048, N=4096, seed=1240)
    inp = workloads.make_inputs(w)
    mean, rstd = _stats(w, inp)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    m, r = torch.from_numpy(mean).to(DEV), torch.from_numpy(rstd).to(DEV)
    first = None
    for _ in range(10):
        outs = rn.ln_backward(dev["dy"], dev["x"], m, r, dev["gamma"])
        torch.cuda.synchronize()
        outs = [o.clone() for o in outs]
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_backward_argument_errors():
    x = torch.zeros(4, 64, device=DEV)
    s = torch.ones(4, device=DEV)
    with pytest.raises(rn.RowNormError) as e:
        rn.ln_backward(x, x, s, s, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == 8
    # rows split across workgroups keep their segment records in the workspace: needed (and
    # checked) even when only dx is wanted
    with pytest.raises(rn.RowNormError) as e:
        rn.ln_backward(torch.zeros(4, 32768, device=DEV), torch.zeros(4, 32768, device=DEV), s, s,
                       want_dgamma=False, want_dbeta=False, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == 8
