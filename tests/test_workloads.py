"""The input recipe: one round-to-nearest-even from float64 to the I/O dtype (CPU only)."""

import numpy as np
import torch

import workloads


def test_round_once_matches_numpy_half_conversion():
    # numpy converts float64 to float16 directly, with one rounding
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(100000) * 8, rng.standard_normal(1000) * 1e-6, [0.0, -0.0, 6e-8]])
    assert np.array_equal(workloads.round_once(v, "fp16"), v.astype(np.float16).astype(np.float64))
    # float32 as well
    assert np.array_equal(workloads.round_once(v, "fp32"), v.astype(np.float32).astype(np.float64))


def test_round_once_is_not_a_double_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 midpoint between 1 and 1 + 2^-7; through
    # float32 it first lands on the midpoint and then ties to even (1), a single rounding
    # gives 1 + 2^-7
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -30, -(1 + 2.0 ** -8 + 2.0 ** -30), 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])
    assert list(workloads.round_once(v, "bf16")) == [1 + 2.0 ** -7, -(1 + 2.0 ** -7), 1.0, 1 + 2 * 2.0 ** -7]
    twice = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert twice[0] == 1.0  # what the two-step conversion would give
    # the same for fp16 (11 bits): 1 + 2^-11 + 2^-30
    v = np.array([1 + 2.0 ** -11 + 2.0 ** -30])
    assert workloads.round_once(v, "fp16")[0] == 1 + 2.0 ** -10


def test_round_once_subnormal_spacing():
    # below the smallest normal the spacing stays the subnormal one
    assert workloads.round_once(np.array([1.4 * 2.0 ** -24]), "fp16")[0] == 2.0 ** -24
    assert workloads.round_once(np.array([2.5 * 2.0 ** -24]), "fp16")[0] == 2 * 2.0 ** -24  # tie to even
    assert workloads.round_once(np.array([1.5 * 2.0 ** -133]), "bf16")[0] == 2 * 2.0 ** -133


def test_inputs_are_exact_in_their_dtype():
    w = workloads.C4_BF16.scaled(rows=4, N=256)
    inp = workloads.make_inputs(w)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    wt = rng.uniform(w.param_lo, w.param_hi, size=w.N)
    assert np.array_equal(inp["weight"].double().numpy(), workloads.round_once(wt, "bf16"))
