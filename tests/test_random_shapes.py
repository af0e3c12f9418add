"""Seeded random sweep over shapes and placements, every case against the fp64 oracle on the
GPU: ops, dtypes, row counts, row lengths from 1 to 70000 elements (every variant's range:
wave, workgroup, 128 KiB workgroup, element and pair, split rows of whole chunks and of
elements), element offsets of the row tensors and padded row strides. The outputs are
checked to the same bars as the targeted parity tests, and nothing outside the output rows
may be written (NaN guards)."""

import numpy as np
import pytest

import workloads
from test_parity import BASES, ROW_TENSORS, check_outputs, run_oracle, run_placed

pytestmark = pytest.mark.gpu

OPS = ["ln", "rms", "fused_add_rms", "fused_add_ln", "softmax"]
DTYPES = ["fp32", "fp16", "bf16"]


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        op, dtype = OPS[rng.integers(len(OPS))], DTYPES[rng.integers(len(DTYPES))]
        band = rng.integers(4)
        lo, hi = [(1, 64), (65, 4096), (4097, 16384), (16385, 70000)][band]
        N = int(rng.integers(lo, hi + 1))
        if rng.random() < 0.3:  # whole 16-byte chunks
            e = 4 if dtype == "fp32" else 8
            N = max(e, N // e * e)
        rows = int(rng.choice([1, 2, 3, 5, 8, 13, 33] if band < 3 else [1, 2, 3]))
        names = ROW_TENSORS if op.startswith("fused") else ("x", "y")
        kind = rng.integers(3)
        if kind == 0:  # dense
            off, ld = None, None
        elif kind == 1:  # one offset for every row tensor, padded strides
            o, p = int(rng.integers(0, 8)), int(rng.integers(0, 10))
            off, ld = {n: o for n in names}, {n: N + p for n in names}
        else:  # independent offsets and strides
            off = {n: int(rng.integers(0, 8)) for n in names}
            ld = {n: N + int(rng.integers(0, 10)) for n in names}
        out.append((i, op, dtype, rows, N, off, ld))
    return out


@pytest.mark.parametrize("case", _cases(400, 2024), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}")
def test_random_shape(case):
    i, op, dtype, rows, N, off, ld = case
    w = BASES[op].scaled(rows=rows, N=N, seed=5000 + i, dtype=dtype)
    inp = workloads.make_inputs(w)
    ref = run_oracle(w, inp)
    out = run_placed(w, inp, offset=off, ld=ld)
    check_outputs(w, ref, *out)


def _bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        op, dtype = ["ln_bwd", "rms_bwd"][rng.integers(2)], DTYPES[rng.integers(len(DTYPES))]
        band = rng.integers(4)
        lo, hi = [(1, 64), (65, 4096), (4097, 16384), (16385, 70000)][band]
        N = int(rng.integers(lo, hi + 1))
        if rng.random() < 0.4:
            e = 4 if dtype == "fp32" else 8
            N = max(e, N // e * e)
        rows = int(rng.choice([1, 2, 3, 7, 40, 300] if band < 2 else [1, 2, 5, 24]))
        out.append((i, op, dtype, rows, N, bool(rng.random() < 0.8), bool(rng.random() < 0.3),
                    bool(rng.random() < 0.85)))
    return out


@pytest.mark.parametrize("case", _bwd_cases(160, 2025), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}")
def test_random_backward(case):
    from test_backward import run_case

    i, op, dtype, rows, N, with_gamma, in_place, params = case
    base = workloads.LN_BWD if op == "ln_bwd" else workloads.RMS_BWD
    run_case(base.scaled(rows=rows, N=N, seed=6000 + i, dtype=dtype), with_gamma=with_gamma, in_place=in_place,
             params=params)
