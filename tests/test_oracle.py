"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix: exact
rational arithmetic on tiny rows, closed forms, invariants of the definitions, library
routines that compute the same textbook quantity (torch's CPU float64 layer_norm and
rms_norm, numpy's float64 -> float16 rounding, torch's float32 -> bfloat16 rounding),
and every bit pattern of the 16-bit formats. A plausible mistake in the oracle (a dropped
eps, unbiased variance, a sign, swapped gamma / beta, squaring the unrounded residual sum,
a wrong rounding tie) fails at least one test here.
"""

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------------------------
# Codec: IEEE fp16 / bf16 / fp32, round-to-nearest-even.
# ------------------------------------------------------------------------------------

def test_decode_every_fp16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_every_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_fp32_patterns():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000, 0xFF800000,
                        0x7FC00000, 0x3F800000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    got = oracle.decode(bits, "fp32")
    with np.errstate(invalid="ignore"):
        ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_encode_roundtrips_every_pattern(dtype):
    bits = np.arange(1 << 16, dtype=np.uint16)
    vals = oracle.decode(bits, dtype)
    keep = ~np.isnan(vals)
    assert np.array_equal(oracle.encode(vals[keep], dtype), bits[keep])


def _finite_sorted_grid(dtype):
    """All finite non-negative values of a 16-bit format, ascending, with their bits."""
    bits = np.arange(0, 1 << 15, dtype=np.uint16)  # sign bit clear
    vals = oracle.decode(bits, dtype)
    keep = np.isfinite(vals)
    return bits[keep], vals[keep]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_encode_ties_go_to_even(dtype):
    # Exact midpoints between consecutive finite values must round to the neighbour with
    # an even last fraction bit.
    bits, vals = _finite_sorted_grid(dtype)
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in fp64
    even_lo = (bits[:-1] & 1) == 0
    expected = np.where(even_lo, bits[:-1], bits[1:])
    assert np.array_equal(oracle.encode(mids, dtype), expected)
    assert np.array_equal(oracle.encode(-mids, dtype), expected | 0x8000)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_encode_is_nearest_by_brute_force(dtype):
    # Random doubles (not representable in fp32 in general): the result must be one of
    # the two bracketing grid values and the nearer one.
    bits, vals = _finite_sorted_grid(dtype)
    rng = np.random.default_rng(11)
    top = vals[-1]
    x = np.concatenate([rng.uniform(0, 1, 20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        rng.uniform(0, top, 2000)])
    got = oracle.encode(x, dtype)
    idx = np.searchsorted(vals, x, side="right") - 1
    lo, hi = vals[idx], vals[np.minimum(idx + 1, len(vals) - 1)]
    dlo, dhi = x - lo, hi - x
    exp = np.where(dlo < dhi, bits[idx], bits[np.minimum(idx + 1, len(vals) - 1)])
    tie = dlo == dhi
    exp = np.where(tie, np.where((bits[idx] & 1) == 0, bits[idx], bits[np.minimum(idx + 1, len(vals) - 1)]), exp)
    assert np.array_equal(got, exp)


def test_encode_fp16_matches_numpy_from_float64():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100_000) * 10.0 ** rng.integers(-8, 5, 100_000)
    x = np.concatenate([x, [65519.0, 65520.0, 65504.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26, 0.0, -0.0]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode(x, "fp16"), ref)


def test_encode_bf16_matches_torch_from_float32():
    rng = np.random.default_rng(4)
    x32 = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-30, 30, 100_000)).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode(x32.astype(np.float64), "bf16"), ref)


def test_encode_fp32_matches_c_cast():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(100_000) * 10.0 ** rng.integers(-40, 38, 100_000)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(oracle.encode(x, "fp32"), ref)


def test_encode_overflow_and_specials():
    # fp16: 65504 is the largest finite value; 65520 is the midpoint to 2^16 and rounds
    # to infinity (the even neighbour).
    assert oracle.encode(np.array([65519.99]), "fp16")[0] == 0x7BFF
    assert oracle.encode(np.array([65520.0]), "fp16")[0] == 0x7C00
    assert oracle.encode(np.array([np.inf, -np.inf]), "bf16").tolist() == [0x7F80, 0xFF80]
    assert np.isnan(oracle.decode(oracle.encode(np.array([np.nan]), "bf16"), "bf16")[0])


# ------------------------------------------------------------------------------------
# Moments: two-pass vs Welford vs exact rationals.
# ------------------------------------------------------------------------------------

def _exact_moments(xs):
    fr = [Fraction(v) for v in xs]
    mean = sum(fr) / len(fr)
    var = sum((v - mean) ** 2 for v in fr) / len(fr)  # biased: 1/N
    return mean, var


@pytest.mark.parametrize("xs", [
    [1.0, 2.0, 3.0, 4.0],
    [0.5, -0.25, 3.75],
    [7.0],
    [-3.0, 5.0],
    [1000.125, 999.875, 1000.5, 999.5, 1000.0, 1000.25, 999.75],
    [2.0 ** -10, 3 * 2.0 ** -12, -(2.0 ** -9), 5 * 2.0 ** -11, 0.0, 1.0],
])
def test_moments_exact_on_tiny_rows(xs):
    mean, var = _exact_moments(xs)
    m_tp, v_tp = oracle.twopass_var(np.array(xs))
    m_w, v_w = oracle.welford_var(np.array(xs))
    for m, v in ((m_tp, v_tp), (m_w, v_w)):
        assert abs(Fraction(m) - mean) <= abs(mean) * Fraction(1, 10 ** 15) + Fraction(1, 10 ** 300)
        assert abs(Fraction(v) - var) <= var * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


def test_twopass_and_welford_agree_on_offset_rows():
    inp = workloads.make_inputs(workloads.C2)
    x = inp["x"].double().numpy()
    for r in range(0, 128, 7):
        m1, v1 = oracle.twopass_var(x[r])
        m2, v2 = oracle.welford_var(x[r])
        assert abs(v1 - v2) <= 1e-12 * v1
        assert abs(m1 - m2) <= 1e-12 * abs(m1)


def test_constant_row_has_zero_variance():
    for c in (1000.1, 3.3, -777.7, 0.1):
        x = np.full(1024, np.float32(c), dtype=np.float64)
        assert oracle.twopass_var(x)[1] == 0.0
        assert oracle.welford_var(x)[1] == 0.0


# ------------------------------------------------------------------------------------
# LayerNorm.
# ------------------------------------------------------------------------------------

getcontext().prec = 60


def _exact_ln_row(xs, g, b, eps):
    mean, var = _exact_moments(xs)
    rstd = 1 / (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(eps)).sqrt()
    ys = []
    for x, gj, bj in zip(xs, g, b):
        d = Fraction(x) - mean
        ys.append(Decimal(d.numerator) / Decimal(d.denominator) * rstd * Decimal(gj) + Decimal(bj))
    return mean, rstd, ys


@pytest.mark.parametrize("row", [
    [1.0, 2.0, 3.0, 4.0],
    [0.5, -0.25, 3.75, 8.0, -1.0],
    [1000.125, 999.875, 1000.5, 999.5, 1000.0, 1000.25, 999.75],
])
def test_layer_norm_matches_exact_arithmetic(row):
    N = len(row)
    g = [0.5 + 0.25 * j for j in range(N)]
    b = [0.125 * (j - 2) for j in range(N)]
    eps = 2.0 ** -17
    x = torch.tensor([row], dtype=torch.float32)
    out = oracle.layer_norm(x, torch.tensor(g, dtype=torch.float32), torch.tensor(b, dtype=torch.float32), eps)
    mean, rstd, ys = _exact_ln_row(row, g, b, eps)
    assert abs(Fraction(out["mean"][0]) - mean) <= abs(mean) * Fraction(1, 10 ** 15)
    assert abs(Decimal(out["rstd"][0]) - rstd) <= rstd * Decimal("1e-15")
    for j in range(N):
        assert abs(Decimal(out["y"][0, j]) - ys[j]) <= Decimal("1e-14") * (1 + abs(ys[j]))


@pytest.mark.parametrize("dtype,rows,N", [("fp32", 13, 1000), ("fp16", 7, 333), ("bf16", 5, 4096), ("fp32", 3, 1)])
def test_layer_norm_matches_torch_float64(dtype, rows, N):
    w = workloads.C1.scaled(rows=rows, N=N, seed=77, dtype=dtype)
    inp = workloads.make_inputs(w)
    eps = 1e-5
    out = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], eps)
    ref = F.layer_norm(inp["x"].double(), (N,), inp["gamma"].double(), inp["beta"].double(), eps).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    xd = inp["x"].double()
    var = xd.var(dim=1, unbiased=False)
    assert np.allclose(out["mean"], xd.mean(dim=1).numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(out["rstd"], (1.0 / torch.sqrt(var + eps)).numpy(), rtol=1e-12)


def test_layer_norm_optional_affine_defaults():
    inp = workloads.make_inputs(workloads.C1.scaled(rows=4, N=64, seed=9))
    base = oracle.layer_norm(inp["x"], None, None, 1e-5)["y"]
    ref = F.layer_norm(inp["x"].double(), (64,), None, None, 1e-5).numpy()
    assert np.allclose(base, ref, rtol=1e-12, atol=1e-12)
    only_g = oracle.layer_norm(inp["x"], inp["gamma"], None, 1e-5)["y"]
    assert np.allclose(only_g, ref * inp["gamma"].double().numpy(), rtol=1e-12, atol=1e-12)
    only_b = oracle.layer_norm(inp["x"], None, inp["beta"], 1e-5)["y"]
    assert np.allclose(only_b, ref + inp["beta"].double().numpy(), rtol=1e-12, atol=1e-12)


def test_layer_norm_closed_form_n1_n2():
    eps = 1e-5
    # N = 1: the deviation is 0, so y = beta, mean = x, rstd = 1/sqrt(eps).
    x = torch.tensor([[3.5], [-1000.25]], dtype=torch.float32)
    g = torch.tensor([1.25], dtype=torch.float32)
    b = torch.tensor([-0.375], dtype=torch.float32)
    out = oracle.layer_norm(x, g, b, eps)
    assert np.all(out["y"] == -0.375)
    assert out["mean"].tolist() == [3.5, -1000.25]
    assert np.allclose(out["rstd"], 1 / math.sqrt(eps), rtol=1e-15)
    # N = 2: y_j = gamma_j * (+-d) / sqrt(d^2 + eps) + beta_j with d = (x0 - x1) / 2.
    x = torch.tensor([[3.0, 1.5]], dtype=torch.float32)
    g = torch.tensor([2.0, 0.5], dtype=torch.float32)
    b = torch.tensor([0.25, -0.75], dtype=torch.float32)
    out = oracle.layer_norm(x, g, b, eps)
    d = (3.0 - 1.5) / 2
    s = math.sqrt(d * d + eps)
    assert np.allclose(out["y"][0], [2.0 * d / s + 0.25, 0.5 * (-d) / s - 0.75], rtol=1e-15)


def test_layer_norm_constant_rows_give_beta_exactly():
    w = workloads.C2.scaled(rows=6, N=1024, seed=21, x_dist="constant")
    inp = workloads.make_inputs(w)
    out = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], 1e-5)
    beta = inp["beta"].double().numpy()
    assert np.array_equal(out["y"], np.broadcast_to(beta, out["y"].shape))
    assert np.allclose(out["rstd"], 1 / math.sqrt(1e-5), rtol=1e-15)


def test_layer_norm_output_moments():
    # With gamma = 1 and beta = 0: per-row mean(y) = 0 and var(y) = var / (var + eps).
    inp = workloads.make_inputs(workloads.C1.scaled(rows=16, N=4096, seed=31))
    eps = 1e-2  # large enough for var / (var + eps) to differ visibly from 1
    out = oracle.layer_norm(inp["x"], None, None, eps)
    y = out["y"]
    var = 1 / out["rstd"] ** 2 - eps
    assert np.all(np.abs(y.mean(axis=1)) <= 1e-13)
    assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_layer_norm_translation_and_scale_laws():
    rng = np.random.default_rng(8)
    x = (rng.integers(-512, 512, size=(4, 256)) / 8.0).astype(np.float32)  # exact dyadics
    g = torch.from_numpy(rng.uniform(0.5, 1.5, 256).astype(np.float32))
    b = torch.from_numpy((0.1 * rng.standard_normal(256)).astype(np.float32))
    eps = 1e-5
    base = oracle.layer_norm(torch.from_numpy(x), g, b, eps)["y"]
    shifted = oracle.layer_norm(torch.from_numpy(x + np.float32(1024.0)), g, b, eps)["y"]
    assert np.allclose(shifted, base, rtol=0, atol=1e-13)
    scaled = oracle.layer_norm(torch.from_numpy(x * np.float32(8.0)), g, b, eps * 64.0)["y"]
    assert np.allclose(scaled, base, rtol=0, atol=1e-13)


def test_layer_norm_threads_are_bitwise_identical():
    inp = workloads.make_inputs(workloads.C2)
    a = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], 1e-5, threads=1)
    b = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], 1e-5, threads=5)
    for k in ("y", "mean", "rstd"):
        assert np.array_equal(a[k], b[k])


def test_offset_config_defeats_naive_moments():
    # The row-offset config is a real cancellation test: variance taken as
    # E[x^2] - E[x]^2 in fp32 misses the oracle by far more than the 1e-4 fp32 bound,
    # while a shifted two-pass in fp32 stays far inside it.
    inp = workloads.make_inputs(workloads.C2)
    ref = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], 1e-5)["y"]
    x = inp["x"].numpy()
    g, b = inp["gamma"].numpy(), inp["beta"].numpy()
    n = np.float32(x.shape[1])
    s = x.sum(axis=1, dtype=np.float32)
    s2 = (x * x).sum(axis=1, dtype=np.float32)
    mean = s / n
    var = np.maximum(s2 / n - mean * mean, np.float32(0))
    y_naive = (x - mean[:, None]) / np.sqrt(var[:, None] + np.float32(1e-5)) * g + b
    assert np.abs(y_naive - ref).max() > 1e-2
    k = x[:, :1]
    d = x - k
    m = d.sum(axis=1, dtype=np.float32, keepdims=True) / n
    v = ((d - m) ** 2).sum(axis=1, dtype=np.float32, keepdims=True) / n
    y_shift = (d - m) / np.sqrt(v + np.float32(1e-5)) * g + b
    assert np.abs(y_shift - ref).max() < 1e-5


def test_layer_norm_rejects_bad_arguments():
    x = torch.zeros(2, 4)
    with pytest.raises(oracle.OracleError):
        oracle.layer_norm(x, None, None, -1.0)


# ------------------------------------------------------------------------------------
# RMSNorm and fused add + RMSNorm.
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,rows,N", [("fp32", 9, 1000), ("fp16", 16, 4096), ("bf16", 4, 255)])
def test_rms_norm_matches_torch_float64(dtype, rows, N):
    w = workloads.C3.scaled(rows=rows, N=N, seed=5, dtype=dtype)
    inp = workloads.make_inputs(w)
    out = oracle.rms_norm(inp["x"], inp["weight"], 1e-6)
    ref = F.rms_norm(inp["x"].double(), (N,), inp["weight"].double(), 1e-6).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)
    xd = inp["x"].double()
    assert np.allclose(out["rstd"], (1 / torch.sqrt((xd * xd).mean(dim=1) + 1e-6)).numpy(), rtol=1e-12)


def test_rms_norm_closed_form_and_invariants():
    eps = 1e-6
    x = torch.tensor([[3.0], [-0.5]], dtype=torch.float32)
    out = oracle.rms_norm(x, torch.tensor([2.0]), eps)
    assert np.allclose(out["y"][:, 0], [2 * 3.0 / math.sqrt(9.0 + eps), 2 * -0.5 / math.sqrt(0.25 + eps)], rtol=1e-15)
    inp = workloads.make_inputs(workloads.C3.scaled(rows=8, N=2048, seed=6))
    eps = 1e-1
    out = oracle.rms_norm(inp["x"], None, eps)
    xd = inp["x"].double().numpy()
    ms = (xd * xd).mean(axis=1)
    assert np.allclose((out["y"] ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-12)
    wt = inp["weight"]
    yw = oracle.rms_norm(inp["x"], wt, 1e-6)["y"]
    assert np.array_equal(np.sign(yw), np.sign(xd) * np.sign(wt.double().numpy()))
    # Scale law: RMS(a x; a^2 eps) = RMS(x; eps) for a power of two a.
    xs = inp["x"].float() * 4.0
    a = oracle.rms_norm(inp["x"].float(), None, 1e-6)["y"]
    b = oracle.rms_norm(xs, None, 16e-6)["y"]
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("w", [workloads.C4_FP16, workloads.C4_BF16], ids=["fp16", "bf16"])
def test_fused_add_rms_norm_semantics(w):
    inp = workloads.make_inputs(w.scaled(rows=32))
    out = oracle.fused_add_rms_norm(inp["x"], inp["residual"], inp["weight"], w.eps)
    td = torch.__dict__["float16" if w.dtype == "fp16" else "bfloat16"]
    # residual_out: the exact sum rounded once to the I/O dtype. fp32 addition of two
    # 16-bit values followed by rounding to 16 bits is correctly rounded (24 >= 2p + 2).
    t = (inp["x"].float() + inp["residual"].float()).to(td)
    assert np.array_equal(out["residual_out"], t.view(torch.int16).numpy().view(np.uint16))
    # y: RMSNorm of the rounded residual stream, not of the unrounded sum.
    ref = F.rms_norm(t.double(), (w.N,), inp["weight"].double(), w.eps).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)
    unrounded = inp["x"].double() + inp["residual"].double()
    rstd_unrounded = (1 / torch.sqrt((unrounded ** 2).mean(dim=1) + w.eps)).numpy()
    if w.dtype == "bf16":
        # the distinction is visible at the 1e-5 rstd bound
        assert np.abs(out["rstd"] / rstd_unrounded - 1).max() > 1e-5


# ------------------------------------------------------------------------------------
# Byte accounting against the pages' printed traffic figures.
# ------------------------------------------------------------------------------------

def test_algorithmic_bytes_match_pages_figures():
    with open(os.path.join(HERE, "golden", "pages_traffic_figures.json")) as f:
        gold = json.load(f)
    for e in gold["effective_bandwidth"]:
        b = workloads.algorithmic_bytes(e["op"], e["rows"], e["N"], 4, with_params=False)
        implied_ms = b / (e["gb_per_s"] * 1e9) * 1e3
        assert round(implied_ms, e["time_decimals"]) == pytest.approx(e["time_ms"]), e["cite"]
    for e in gold["dram_traffic"]:
        x_bytes = e["rows"] * e["N"] * 4
        if e["op"] == "ln":
            assert x_bytes == e["x_mib"] * 2 ** 20
            b = workloads.algorithmic_bytes("ln", e["rows"], e["N"], 4)
            assert e["ideal_mib_floor"] * 2 ** 20 < b < e["ideal_mib_ceil"] * 2 ** 20
        else:
            two_kernel = 3 * x_bytes + 2 * e["N"] * 4 + 2 * 2 * e["rows"] * 4
            assert abs(two_kernel / 2 ** 20 - e["total_mib_approx"]) < 1.0


# ------------------------------------------------------------------------------------
# Fused residual add + LayerNorm.
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_fused_add_layer_norm_semantics(dtype):
    w = workloads.FUSED_LN.scaled(rows=24, N=512, dtype=dtype)
    inp = workloads.make_inputs(w)
    out = oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp["gamma"], inp["beta"], w.eps)
    td = workloads.TORCH_DTYPES[dtype]
    # residual_out: the exact sum rounded once (for 16-bit inputs fp32 addition then
    # rounding is correctly rounded; for fp32 the exact sum is formed in fp64 and rounded).
    if dtype == "fp32":
        t = (inp["x"].double() + inp["residual"].double()).float()
        bits = t.view(torch.int32).numpy().view(np.uint32)
    else:
        t = (inp["x"].float() + inp["residual"].float()).to(td)
        bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out["residual_out"], bits)
    # y, mean, rstd: torch's float64 LayerNorm of the rounded stream
    ref = F.layer_norm(t.double(), (w.N,), inp["gamma"].double(), inp["beta"].double(), w.eps).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    td64 = t.double()
    assert np.allclose(out["mean"], td64.mean(dim=1).numpy(), rtol=1e-13, atol=1e-13)
    var = td64.var(dim=1, unbiased=False)
    assert np.allclose(out["rstd"], (1 / torch.sqrt(var + w.eps)).numpy(), rtol=1e-12)
    # the plain LayerNorm of the rounded stream is the same computation
    plain = oracle.layer_norm(t, inp["gamma"], inp["beta"], w.eps)
    assert np.array_equal(plain["y"], out["y"])


def test_fused_add_layer_norm_uses_the_rounded_sum():
    # bf16: x + residual is not representable; normalizing the unrounded sum differs
    w = workloads.FUSED_LN.scaled(rows=16, N=256)
    inp = workloads.make_inputs(w)
    out = oracle.fused_add_layer_norm(inp["x"], inp["residual"], inp["gamma"], inp["beta"], w.eps)
    exact = (inp["x"].double() + inp["residual"].double())
    ref_unrounded = F.layer_norm(exact, (w.N,), inp["gamma"].double(), inp["beta"].double(), w.eps).numpy()
    assert np.abs(out["y"] - ref_unrounded).max() > 1e-4


# ------------------------------------------------------------------------------------
# Softmax.
# ------------------------------------------------------------------------------------

def _exact_softmax(xs):
    getcontext().prec = 50
    d = [Decimal(v) for v in xs]
    m = max(d)
    e = [(v - m).exp() for v in d]
    s = sum(e)
    return [float(v / s) for v in e], float(s)


@pytest.mark.parametrize("xs", [
    [0.0], [1.0, 2.0], [-3.5, 0.25, 7.0], [1.0, 1.0, 1.0, 1.0, 1.0],
    [100.0, -100.0, 0.5, 0.75, -0.125, 3.0, 2.0],
])
def test_softmax_matches_50_digit_arithmetic(xs):
    x = torch.tensor([xs], dtype=torch.float32)
    out = oracle.softmax(x)
    ref, s = _exact_softmax(xs)
    assert np.allclose(out["y"][0], ref, rtol=1e-15, atol=1e-300)
    assert out["max"][0] == max(xs)
    assert out["sum"][0] == pytest.approx(s, rel=1e-15)


@pytest.mark.parametrize("dtype,rows,N", [("fp32", 8, 4096), ("fp16", 5, 333), ("bf16", 3, 1000)])
def test_softmax_matches_scipy_float64(dtype, rows, N):
    from scipy.special import softmax as sp_softmax

    inp = workloads.make_inputs(workloads.SOFTMAX.scaled(rows=rows, N=N, dtype=dtype, seed=5))
    out = oracle.softmax(inp["x"])
    ref = sp_softmax(inp["x"].double().numpy(), axis=1)
    assert np.allclose(out["y"], ref, rtol=1e-13, atol=0)
    assert np.allclose(out["y"].sum(axis=1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_softmax_masked_entries(dtype):
    # entries of -inf (masked logits) take no part: the softmax of a masked row is scipy's
    # float64 softmax of its other entries, with exact zeros where masked; leading runs of
    # -inf (where the online form's rescaling is undefined) included
    from scipy.special import softmax as sp_softmax

    inp = workloads.make_inputs(workloads.SOFTMAX.scaled(rows=6, N=300, dtype=dtype, seed=11))
    x = inp["x"].clone()
    rng = np.random.default_rng(12)
    mask = rng.random(x.shape) < 0.4
    mask[1, :37] = True  # a leading run
    mask[2, 150:] = True  # a trailing run
    mask[3, :] = False
    mask[3, 299] = True
    x[torch.from_numpy(mask)] = float("-inf")
    out = oracle.softmax(x)
    for r in range(x.shape[0]):
        keep = ~mask[r]
        ref = np.zeros(x.shape[1])
        ref[keep] = sp_softmax(x[r].double().numpy()[keep])
        assert np.allclose(out["y"][r], ref, rtol=1e-13, atol=0)
        assert np.all(out["y"][r][mask[r]] == 0.0)
        assert out["max"][r] == x[r].double().numpy()[keep].max()
    # no entry above -inf: no softmax (NaN outputs), maximum -inf, sum 0
    z = torch.full((2, 9), float("-inf"), dtype=x.dtype)
    o = oracle.softmax(z)
    assert np.all(np.isnan(o["y"])) and np.all(o["max"] == -np.inf) and np.all(o["sum"] == 0.0)


def test_softmax_closed_forms_and_invariants():
    # two elements: the logistic function of the difference
    x = torch.tensor([[2.0, -1.0], [0.0, 0.0], [-5.0, 5.0]], dtype=torch.float32)
    y = oracle.softmax(x)["y"]
    d = (x[:, 0] - x[:, 1]).double().numpy()
    assert np.allclose(y[:, 0], 1 / (1 + np.exp(-d)), rtol=1e-15)
    # constant rows: exactly 1 / N
    c = torch.full((3, 12), 7.25)
    assert np.all(oracle.softmax(c)["y"] == 1.0 / 12)
    # shift invariance (the shift is exact in fp32 for these dyadic values)
    z = torch.tensor([[0.5, -2.25, 3.0, 1.0, -0.75]])
    a = oracle.softmax(z)["y"]
    b = oracle.softmax(z + 64.0)["y"]
    assert np.allclose(a, b, rtol=1e-15, atol=0)
    # order is preserved and every output lies in (0, 1]
    assert list(np.argsort(a[0])) == list(np.argsort(z[0].numpy()))
    assert np.all(a > 0) and np.all(a <= 1)
    # large logits do not overflow: the maximum is subtracted first
    big = torch.tensor([[1000.0, 999.0, -1000.0]])
    yb = oracle.softmax(big)["y"][0]
    assert np.isfinite(yb).all() and yb[0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)


# ------------------------------------------------------------------------------------
# Backward passes.
# ------------------------------------------------------------------------------------

def _central_difference(f, x, h):
    """Gradient of the scalar function f at x by central differences, one coordinate at a time."""
    g = np.empty_like(x)
    for j in range(x.size):
        xp = x.copy(); xp[j] += h
        xm = x.copy(); xm[j] -= h
        g[j] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("N", [1, 2, 7, 40])
def test_layer_norm_backward_is_the_derivative_of_the_forward(N):
    rng = np.random.default_rng(N)
    x = (3.0 + 2.0 * rng.standard_normal(N)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32)
    dy = rng.standard_normal(N).astype(np.float32)
    eps = 1e-3
    out = oracle.layer_norm_backward(torch.from_numpy(dy[None]), torch.from_numpy(x[None]), torch.from_numpy(g),
                                     eps=eps)
    x64, g64, b64, dy64 = (a.astype(np.float64) for a in (x, g, b, dy))
    loss = lambda xx: float(np.dot(dy64, oracle.layer_norm_row_f64(xx, g64, b64, eps)))
    fd = _central_difference(loss, x64, 1e-5)
    assert np.allclose(out["dx"][0], fd, rtol=1e-6, atol=1e-7)
    loss_g = lambda gg: float(np.dot(dy64, oracle.layer_norm_row_f64(x64, gg, b64, eps)))
    assert np.allclose(out["dgamma"], _central_difference(loss_g, g64, 1e-5), rtol=1e-6, atol=1e-7)
    loss_b = lambda bb: float(np.dot(dy64, oracle.layer_norm_row_f64(x64, g64, bb, eps)))
    assert np.allclose(out["dbeta"], _central_difference(loss_b, b64, 1e-5), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("N", [1, 3, 40])
def test_rms_norm_backward_is_the_derivative_of_the_forward(N):
    rng = np.random.default_rng(100 + N)
    x = rng.standard_normal(N).astype(np.float32)
    w = rng.uniform(0.5, 1.5, N).astype(np.float32)
    dy = rng.standard_normal(N).astype(np.float32)
    eps = 1e-3
    out = oracle.rms_norm_backward(torch.from_numpy(dy[None]), torch.from_numpy(x[None]), torch.from_numpy(w), eps=eps)
    x64, w64, dy64 = (a.astype(np.float64) for a in (x, w, dy))
    loss = lambda xx: float(np.dot(dy64, oracle.rms_norm_row_f64(xx, w64, eps)))
    assert np.allclose(out["dx"][0], _central_difference(loss, x64, 1e-5), rtol=1e-6, atol=1e-7)
    loss_w = lambda ww: float(np.dot(dy64, oracle.rms_norm_row_f64(x64, ww, eps)))
    assert np.allclose(out["dweight"], _central_difference(loss_w, w64, 1e-5), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_layer_norm_backward_matches_torch_autograd_float64(dtype):
    w = workloads.LN_BWD.scaled(rows=6, N=300, dtype=dtype)
    inp = workloads.make_inputs(w)
    out = oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"], eps=w.eps)
    x = inp["x"].double().requires_grad_(True)
    g = inp["gamma"].double().requires_grad_(True)
    b = inp["beta"].double().requires_grad_(True)
    F.layer_norm(x, (w.N,), g, b, w.eps).backward(inp["dy"].double())
    assert np.allclose(out["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(out["dgamma"], g.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(out["dbeta"], b.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_rms_norm_backward_matches_torch_autograd_float64():
    w = workloads.RMS_BWD.scaled(rows=5, N=257)
    inp = workloads.make_inputs(w)
    out = oracle.rms_norm_backward(inp["dy"], inp["x"], inp["weight"], eps=w.eps)
    x = inp["x"].double().requires_grad_(True)
    wt = inp["weight"].double().requires_grad_(True)
    F.rms_norm(x, (w.N,), wt, w.eps).backward(inp["dy"].double())
    assert np.allclose(out["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(out["dweight"], wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_invariants_and_given_statistics():
    w = workloads.LN_BWD.scaled(rows=8, N=128, dtype="fp32")
    inp = workloads.make_inputs(w)
    out = oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"], eps=w.eps)
    fwd = oracle.layer_norm(inp["x"], inp["gamma"], inp["beta"], w.eps)
    scale = np.abs(out["dx"]).max()
    # dx is orthogonal to the constant direction (for any eps) ...
    assert np.abs(out["dx"].sum(axis=1)).max() < 1e-12 * scale * w.N
    # ... and, with eps = 0, to xhat: sum_j xhat_j^2 = N exactly cancels the last term
    z = oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"], eps=0.0)
    f0 = oracle.layer_norm(inp["x"], None, None, 0.0)
    xhat = (inp["x"].double().numpy() - f0["mean"][:, None]) * f0["rstd"][:, None]
    assert np.abs((z["dx"] * xhat).sum(axis=1)).max() < 1e-12 * np.abs(z["dx"]).max() * w.N
    # with eps > 0 the same sum is rstd * sum(g * xhat) * eps / (var + eps), not zero
    assert np.abs((out["dx"] * xhat).sum(axis=1)).max() > 1e-9
    # dbeta: the exact column sums of dy (small-integer multiples of fp32 values)
    dyf = [[Fraction(float(v)) for v in row] for row in inp["dy"].tolist()]
    for j in (0, 17, 127):
        assert out["dbeta"][j] == float(sum(r[j] for r in dyf))
    # the forward's fp32 statistics, given explicitly, are used as given: the result
    # moves by about the statistics' rounding, no more
    given = oracle.layer_norm_backward(inp["dy"], inp["x"], inp["gamma"],
                                       mean=fwd["mean"].astype(np.float32), rstd=fwd["rstd"].astype(np.float32),
                                       eps=w.eps)
    d = np.abs(given["dx"] - out["dx"]).max()
    assert 0 < d < 1e-5 * scale
    # RMSNorm with eps = 0: dx is orthogonal to x
    rw = workloads.RMS_BWD.scaled(rows=4, N=96, dtype="fp32")
    ri = workloads.make_inputs(rw)
    ro = oracle.rms_norm_backward(ri["dy"], ri["x"], ri["weight"], eps=0.0)
    xs = ri["x"].double().numpy()
    assert np.abs((ro["dx"] * xs).sum(axis=1)).max() < 1e-12 * np.abs(ro["dx"]).max() * rw.N * np.abs(xs).max()
