"""GPU parity of rows held exactly by row groups of 3 to 15 (odd) chunks per lane: whole-chunk
rows of 64 x 2^k x o chunks (o = 3, 5, ..., 15), such as 16-bit rows of 1536, 2560, 3072, 3584, 5120,
6144, 7168 or 14336 elements and fp32 rows of 5120 or 7168, launched persistent on a row group
of 2^k waves with no idle slot. Every case is checked against the fp64 oracle (the bars of the
other parity tests), the plan is checked to be that row group, and the bytes around every
output row are checked to be left as they were. Cases cover o = 3, 5, 7 on 1, 2, 4 and 8 waves
(o = 3 also on 16; o = 9 to 15 on 1, 2 and 4), every operation, each dtype, with and without parameters, in place, and
padded row strides."""

import pytest

from test_ragged_rows import run_case

pytestmark = pytest.mark.gpu

# (op, dtype, rows, N, waves per row, chunks per lane)
SHAPES = [
    ("ln", "bf16", 1030, 1536, 1, 3),
    ("rms", "fp16", 1027, 2560, 1, 5),
    ("ln", "bf16", 1025, 3584, 1, 7),
    ("softmax", "fp32", 1029, 768, 1, 3),
    ("ln", "fp32", 515, 1536, 2, 3),
    ("fused_add_rms", "bf16", 517, 5120, 2, 5),
    ("fused_add_ln", "fp16", 513, 7168, 2, 7),
    ("softmax", "fp32", 519, 3584, 2, 7),
    ("ln", "bf16", 521, 5120, 2, 5),
    ("rms", "bf16", 515, 7168, 2, 7),
    ("ln", "fp32", 259, 5120, 4, 5),
    ("rms", "bf16", 263, 14336, 4, 7),
    ("fused_add_ln", "bf16", 261, 6144, 4, 3),
    ("fused_add_rms", "fp32", 257, 7168, 4, 7),
    ("ln", "bf16", 258, 20480, 8, 5),
    ("fused_add_rms", "fp16", 260, 28672, 8, 7),
    ("softmax", "bf16", 262, 12288, 8, 3),
    ("ln", "fp32", 257, 14336, 8, 7),
    ("ln", "bf16", 259, 24576, 16, 3),
    ("rms", "fp32", 261, 12288, 16, 3),
    ("ln", "bf16", 1026, 4608, 1, 9),
    ("softmax", "fp32", 1027, 2304, 1, 9),
    ("fused_add_rms", "fp16", 515, 9216, 2, 9),
    ("fused_add_ln", "bf16", 259, 18432, 4, 9),
    ("rms", "fp32", 261, 9216, 4, 9),
    ("ln", "bf16", 1025, 5632, 1, 11),
    ("fused_add_ln", "fp16", 513, 13312, 2, 13),
    ("rms", "bf16", 1027, 7680, 1, 15),
    ("softmax", "fp32", 259, 15360, 4, 15),
    ("ln", "fp32", 257, 11264, 4, 11),
    ("fused_add_rms", "bf16", 1029, 6656, 1, 13),
]


def _check_plan(info, W, V):
    assert info["variant"] in ("wave", "workgroup"), info
    assert (info["waves_per_row"], info["chunks_per_lane"]) == (W, V), info
    assert info["exact"] and info["persistent"] and not info["ragged"], info


@pytest.mark.parametrize("op,dtype,rows,N,W,V", SHAPES, ids=[f"{s[0]}-{s[1]}-{s[2]}x{s[3]}" for s in SHAPES])
def test_odd_depth_rows_against_the_oracle(op, dtype, rows, N, W, V):
    _check_plan(run_case(op, dtype, rows, N, seed=2100 + N % 89), W, V)


@pytest.mark.parametrize("op,dtype,rows,N,W,V,gamma,beta", [
    ("ln", "bf16", 521, 5120, 2, 5, False, False),
    ("ln", "fp16", 1030, 3584, 1, 7, True, False),
    ("ln", "fp32", 259, 5120, 4, 5, False, True),
    ("rms", "bf16", 515, 7168, 2, 7, False, False),
    ("fused_add_ln", "bf16", 261, 6144, 4, 3, True, False),
    ("fused_add_rms", "fp16", 517, 5120, 2, 5, False, False),
])
def test_odd_depth_rows_without_parameters(op, dtype, rows, N, W, V, gamma, beta):
    _check_plan(run_case(op, dtype, rows, N, seed=2150 + N % 83, gamma=gamma, beta=beta), W, V)


@pytest.mark.parametrize("op,dtype,rows,N,W,V", [("ln", "bf16", 521, 5120, 2, 5), ("fused_add_ln", "fp16", 513, 7168, 2, 7),
                                                 ("fused_add_rms", "bf16", 263, 14336, 4, 7),
                                                 ("softmax", "fp32", 1029, 768, 1, 3)])
def test_odd_depth_rows_in_place(op, dtype, rows, N, W, V):
    # y over x (and residual_out over residual): each lane loads its chunks before it stores them
    _check_plan(run_case(op, dtype, rows, N, seed=2190 + rows % 7, in_place=True), W, V)


@pytest.mark.parametrize("op,dtype,rows,N,W,V,ld", [
    ("ln", "bf16", 521, 5120, 2, 5, {"x": 5128, "y": 5136}),
    ("fused_add_rms", "fp32", 257, 7168, 4, 7, {"residual": 7172, "residual_out": 7176}),
])
def test_odd_depth_rows_with_padded_strides(op, dtype, rows, N, W, V, ld):
    # row strides that keep every row 16-byte aligned: the same kernels, rows addressed by stride
    _check_plan(run_case(op, dtype, rows, N, seed=2210 + rows % 11, ld=ld), W, V)
