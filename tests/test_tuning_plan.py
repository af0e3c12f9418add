"""CPU-side tests of the caller-chosen launch plans (rn_tuning, rn_plan_tuned): which tunings
resolve to a built kernel, which are rejected, and what plan they give. Host only: no kernel
is launched."""

import pytest
import torch

import row_wise_normalization_fp32_amd as rn

OK, UNSUP = 0, 5
BF16, F16, F32 = torch.bfloat16, torch.float16, torch.float32
PARAMS = {"gamma": 1 << 44, "beta": (1 << 44) + (1 << 30)}


def plan(op, rows, N, dtype, tuning, **kw):
    return rn.plan(op, rows, N, dtype, ptrs=dict(PARAMS), tuning=tuning, **kw)


def test_empty_and_automatic_tuning_is_the_automatic_plan():
    for t in ({}, {"waves_per_row": 0, "chunks_per_lane": 0, "persistent": -1, "prefetch": -1, "grid_blocks": 0}):
        for args in (("ln", 4096, 16384, BF16), ("fused_add_rms", 8192, 4096, F16), ("softmax", 300, 4096, F32)):
            assert plan(*args, t) == plan(*args, None)


@pytest.mark.parametrize("W,V,rpb,exact", [(1, 8, 4, True), (2, 4, 2, True), (4, 2, 1, True)])
def test_waves_per_row(W, V, rpb, exact):
    # LayerNorm bf16 rows of 4096 elements: 512 chunks, covered exactly by each of these
    st, info = plan("ln", 8192, 4096, BF16, {"waves_per_row": W})
    assert st == OK
    assert (info["waves_per_row"], info["chunks_per_lane"], info["rows_per_block"]) == (W, V, rpb)
    assert info["variant"] == ("wave" if W == 1 else "workgroup")
    assert info["block_threads"] == 64 * W * rpb and info["exact"] == exact
    assert info["persistent"] and info["grid_blocks"] == 8192 // rpb


def test_unbuilt_shapes_are_unsupported():
    # no kernel of 8 waves x 1 chunk, 16 waves x 2 chunks, or 2 waves x 8 chunks is built
    assert plan("ln", 8192, 4096, BF16, {"waves_per_row": 8})[0] == UNSUP
    assert plan("ln", 4096, 16384, BF16, {"waves_per_row": 16})[0] == UNSUP
    assert plan("ln", 4096, 8192, BF16, {"waves_per_row": 2})[0] == UNSUP
    # 16 waves x 4 chunks covers 16384 bf16 elements twice over: built for grid-per-row
    # launches only (persistent launches need rows that exactly fill the row group)
    st, info = plan("ln", 4096, 16384, BF16, {"waves_per_row": 16, "chunks_per_lane": 4, "persistent": 0})
    assert st == OK and not info["exact"] and not info["persistent"]
    assert plan("ln", 4096, 16384, BF16, {"waves_per_row": 16, "chunks_per_lane": 4, "persistent": 1})[0] == UNSUP


def test_invalid_tunings():
    for t in ({"waves_per_row": 3}, {"waves_per_row": 32}, {"waves_per_row": -1}, {"chunks_per_lane": -1},
              {"chunks_per_lane": 65}, {"persistent": 2}, {"prefetch": 2}, {"grid_blocks": -5}):
        assert plan("ln", 8192, 4096, BF16, t)[0] == UNSUP, t
    # chunks per lane that do not cover the row
    assert plan("ln", 8192, 4096, BF16, {"chunks_per_lane": 2})[0] == UNSUP
    with pytest.raises(ValueError):
        plan("ln", 8192, 4096, BF16, {"waves": 2})


def test_tuning_applies_to_vectorized_variants_only():
    # few ragged rows (element / pair kernels), split rows and the general kernel take no tuning
    assert plan("ln", 300, 4095, BF16, {"grid_blocks": 64})[0] == UNSUP
    assert plan("ln", 64, 65536, F32, {"grid_blocks": 64}, workspace_bytes=1 << 24)[0] == UNSUP
    assert plan("ln", 64, 64, F32, {"persistent": 0}, variant="general")[0] == UNSUP
    # ... but an all-automatic tuning is accepted everywhere
    assert plan("ln", 8192, 4095, BF16, {})[0] == OK


def test_persistent_prefetch_and_grid():
    # LayerNorm bf16 4096 x 16384 with gamma and beta: 8 waves per row, both persistent
    # instances built (rows of 4 or more waves with parameters)
    for pf in (0, 1):
        st, info = plan("ln", 4096, 16384, BF16, {"prefetch": pf, "grid_blocks": 512})
        assert st == OK and info["persistent"] and info["grid_blocks"] == 512
    # the grid is capped at the row blocks
    assert plan("ln", 4096, 16384, BF16, {"grid_blocks": 1 << 20})[1]["grid_blocks"] == 4096
    # without parameters, or with 2 waves per row, only the prefetching instance is built
    assert rn.plan("ln", 4096, 16384, BF16, tuning={"prefetch": 0})[0] == UNSUP
    assert plan("ln", 8192, 4096, BF16, {"prefetch": 0})[0] == UNSUP
    assert plan("ln", 8192, 4096, BF16, {"prefetch": 1, "grid_blocks": 300})[0] == OK
    # one-wave rows of 8 chunks per lane have only the looping instance
    assert plan("ln", 8192, 4096, BF16, {"waves_per_row": 1, "prefetch": 1})[0] == UNSUP
    assert plan("ln", 8192, 4096, BF16, {"waves_per_row": 1, "prefetch": 0})[0] == OK
    # a prefetch choice needs a persistent launch
    assert plan("ln", 8192, 4096, BF16, {"persistent": 0, "prefetch": 1})[0] == UNSUP


def test_launch_mode():
    # grid per row instead of persistent, and the reverse below the persistent threshold
    st, info = plan("ln", 8192, 4096, BF16, {"persistent": 0})
    assert st == OK and not info["persistent"] and info["lds_bytes"] == 0
    st, info = plan("ln", 200, 4096, BF16, None)
    assert st == OK and not info["persistent"]
    st, info = plan("ln", 200, 4096, BF16, {"persistent": 1})
    assert st == OK and info["persistent"] and info["lds_bytes"] == 4096 * 2
    # grid-per-row launches with fewer workgroups than row blocks loop over the rest
    st, info = plan("ln", 8192, 4096, BF16, {"persistent": 0, "grid_blocks": 100})
    assert st == OK and info["grid_blocks"] == 100
    # non-exact rows are persistent only as byte-addressed rows (from 256 row blocks)
    assert plan("rms", 500, 1000, F32, {"persistent": 1})[0] == UNSUP
    st, info = plan("rms", 8192, 1000, F32, {"persistent": 1})
    assert st == OK and info["ragged"] and not info["exact"], info


def test_tuned_entry_point_rejects_before_launch():
    # validation failures return before any HIP call: safe without a GPU
    t = rn._tuning({"waves_per_row": 3})
    import ctypes

    st = rn._lib.rn_forward_tuned(0, 0x100000, None, None, None, 0x200000, None, None, None, 4, 4096, 1e-5, 2,
                                  None, 0, ctypes.byref(t), None, 0, None)
    assert st == UNSUP
    t = rn._tuning({"waves_per_row": 8})  # not built for these rows
    st = rn._lib.rn_forward_tuned(0, 0x100000, None, None, None, 0x200000, None, None, None, 4, 4096, 1e-5, 2,
                                  None, 0, ctypes.byref(t), None, 0, None)
    assert st == UNSUP


@pytest.mark.parametrize("op,rows,N,dtype,W,V", [
    ("ln", 16384, 1536, BF16, 1, 3), ("rms", 16384, 2560, F16, 1, 5), ("ln", 16384, 3584, BF16, 1, 7),
    ("ln", 8192, 3072, BF16, 2, 3), ("ln", 8192, 5120, BF16, 2, 5), ("rms", 8192, 7168, BF16, 2, 7),
    ("fused_add_ln", 8192, 6144, BF16, 4, 3), ("ln", 8192, 5120, F32, 4, 5), ("fused_add_rms", 4096, 14336, F16, 4, 7),
    ("softmax", 4096, 12288, BF16, 8, 3), ("ln", 4096, 20480, BF16, 8, 5), ("ln", 4096, 7168 * 2, F32, 8, 7),
    ("ln", 2048, 24576, BF16, 16, 3),
    ("ln", 16384, 4608, BF16, 1, 9), ("ln", 16384, 2304, F32, 1, 9), ("rms", 8192, 9216, F16, 2, 9),
    ("fused_add_ln", 4096, 18432, BF16, 4, 9),
    ("ln", 16384, 5632, BF16, 1, 11), ("ln", 16384, 6656, BF16, 1, 13), ("rms", 16384, 7680, F16, 1, 15),
    ("softmax", 4096, 15360, F32, 4, 15),
])
def test_rows_held_exactly_by_odd_chunk_counts(op, rows, N, dtype, W, V):
    # rows of 64 x W x V chunks, V = 3, 5, 7: W waves with V chunks per lane, exact and
    # persistent, automatically and when the caller names W
    for t in (None, {"waves_per_row": W}, {"waves_per_row": W, "persistent": 1}):
        st, info = plan(op, rows, N, dtype, t)
        assert st == OK, (t, st)
        assert (info["waves_per_row"], info["chunks_per_lane"]) == (W, V), (t, info)
        assert info["exact"] and info["persistent"] and not info["ragged"], (t, info)


def test_odd_chunk_counts_fall_back_where_not_built():
    # few rows (under 256 row blocks of the exact row group): the power-of-two plan
    st, info = plan("ln", 300, 5120, BF16, None)
    assert st == OK and (info["waves_per_row"], info["chunks_per_lane"]) == (4, 4) and info["ragged"], info
    st, info = plan("ln", 100, 5120, BF16, None)
    assert st == OK and not info["persistent"] and not info["exact"], info
    # a caller-chosen grid-per-row launch, or another width: power-of-two chunks per lane
    st, info = plan("ln", 8192, 5120, BF16, {"waves_per_row": 4})
    assert st == OK and (info["chunks_per_lane"], info["exact"], info["persistent"]) == (4, False, False), info
    assert plan("ln", 8192, 5120, BF16, {"waves_per_row": 2, "persistent": 0})[0] == UNSUP  # 2 x 8 not built
    st, info = plan("ln", 8192, 5120, BF16, {"waves_per_row": 1, "persistent": 0})
    assert st == OK and (info["chunks_per_lane"], info["persistent"]) == (16, False), info
    # 17 and 19 chunks per 64 lanes (and 9 at 8 waves): no exact odd row group
    for N in (8704, 9728):
        st, info = plan("ln", 8192, N, BF16, None)
        assert st == OK and info["chunks_per_lane"] in (1, 2, 4) and not info["exact"], (N, info)
    # a caller-chosen odd count on a grid-per-row launch is not built
    assert plan("ln", 8192, 5120, BF16, {"waves_per_row": 2, "chunks_per_lane": 5, "persistent": 0})[0] == UNSUP


def test_byte_addressed_rows_take_launch_tunings():
    # many ragged rows (byte-addressed, persistent): grid size and instance, and widths whose
    # chunks per lane are built (4; 1 or 2 on one wave); never grid per row
    auto = plan("ln", 8192, 4095, BF16, None)[1]
    assert auto["ragged"] and auto["persistent"] and (auto["waves_per_row"], auto["chunks_per_lane"]) == (2, 4)
    for t in ({"grid_blocks": 64}, {"prefetch": 1, "grid_blocks": 1000}, {"persistent": 1}):
        st, info = plan("ln", 8192, 4095, BF16, t)
        assert st == OK and info["ragged"] and info["persistent"], (t, info)
        assert (info["waves_per_row"], info["chunks_per_lane"]) == (2, 4), (t, info)
    st, info = plan("ln", 8192, 4095, BF16, {"grid_blocks": 64})
    assert info["grid_blocks"] == 64
    assert plan("ln", 8192, 4095, BF16, {"persistent": 0})[0] == UNSUP
    assert plan("ln", 8192, 4095, BF16, {"prefetch": 0})[0] == UNSUP  # 2 waves: the prefetching instance only
    st, info = plan("ln", 4096, 16383, BF16, {"prefetch": 0})  # 8 waves with parameters: both instances
    assert st == OK and info["ragged"] and (info["waves_per_row"], info["chunks_per_lane"]) == (8, 4), info
    st, info = plan("ln", 8192, 4095, BF16, {"waves_per_row": 4})  # 4 x 2 chunks: not built
    assert st == UNSUP, info
    st, info = plan("ln", 8192, 4095, BF16, {"waves_per_row": 1})  # 1 x 8 chunks: not built
    assert st == UNSUP, info
