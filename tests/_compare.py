"""Comparison of GPU outputs with the oracle, at the tolerances the parity tests use.

* fp32 outputs: max |y_gpu - y_ref| <= 1e-4 (absolute), y_ref in fp64.
* fp16 / bf16 outputs: at most 2 output ulps from round(y_ref), the oracle's single
  round-to-nearest-even of the fp64 result, with the ulp measured on the format's own grid:
  the spacing at |y_ref|, and below the smallest normal (fp16 2^-14, bf16 2^-126) the
  subnormal spacing (fp16 2^-24, bf16 2^-133). This native bar applies to RMSNorm, fused
  add + RMSNorm and softmax: their outputs are products and quotients (x * rstd * w,
  exp(x - m) / S) whose fp32 evaluation errs by a few fp32 ulps relative to the result,
  far below one 16-bit ulp at any magnitude, so one rounding leaves at most 1 ulp.
  LayerNorm and fused add + LayerNorm alone add beta: where an output crosses zero
  (z * gamma close to -beta) the fp32 sum carries an absolute error of a few fp32 ulps of
  |beta| (about 3e-7 for |beta| near 0.4), which no fp32-accumulating kernel avoids and
  which exceeds the native 2-ulp band at the smallest magnitudes. For these two ops only,
  the ulp is taken at max(|y_ref|, floor_T): floor_bf16 = 2^-14 (spacing 2^-21),
  floor_fp16 = 2^-10 (spacing 2^-20), which puts the band at 9.5e-7 (bf16) and 1.9e-6
  (fp16). Above the floor the native 2-ulp bar applies unchanged.
* mean: |mean_gpu - mean_ref| <= 1e-5 * max(|mean_ref|, sigma_ref), sigma_ref = sqrt(var);
  rstd: |rstd_gpu / rstd_ref - 1| <= 1e-5.
* residual_out: bit-exact.
* softmax y: fp32 |y_gpu - y_ref| <= 1e-5 * y_ref + 2^-126; fp16 / bf16 as above (2 native
  ulps).
  Derivation for fp32: each output is exp(x - m_w) * exp(m_w - m) / S. x - m_w is exact
  near the maximum; the kernel evaluates exp with a split argument (u * log2 e formed
  exactly as hi + lo, 2^n applied by ldexp, v_exp_f32 only on [-0.5, 0.5]), so each
  exponential is within a few ulps relative for every argument (a plain v_exp_f32 of
  u * log2 e loses about |u| * 2^-23 relative: 1e-5 at u = -55). The rescaling and the
  division add a few ulps, and S (per-lane sums of <= 16 terms, a 6-level lane tree, at
  most 16 wave parts) at most (16 + 6 + 16) * 2^-24 = 2.3e-6 relative. The total stays
  below 1e-5; the absolute floor covers results in the subnormal range.
  row_max: bit-exact (a maximum of the inputs); row_sum: relative <= 1e-5.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

FP32_ABS_TOL = 1e-4
ULP_TOL = 2.0
STAT_REL_TOL = 1e-5
MANT_BITS = {"fp16": 10, "bf16": 7}
# Magnitude floor of the ulp for the ops whose outputs can cancel against beta.
CANCEL_FLOOR = {"fp16": 2.0 ** -10, "bf16": 2.0 ** -14}
# The format's own grid: below the smallest normal the spacing stays the subnormal one.
NATIVE_FLOOR = {"fp16": 2.0 ** -14, "bf16": 2.0 ** -126}
CANCELLING_OPS = ("ln", "fused_add_ln")
# For one output ulp of a backward result: below its smallest normal (2^-14) fp16's grid
# keeps the subnormal spacing 2^-24, so the magnitude is floored there; bf16's subnormals
# (below 2^-126) are out of reach, 2^-24 only keeps the logarithm finite.
GRID_FLOOR = {"fp16": 2.0 ** -14, "bf16": 2.0 ** -24}
_NAME = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}


def dtype_name(t: torch.Tensor) -> str:
    return _NAME[t.dtype]


def ulp_distance(got: np.ndarray, ref64: np.ndarray, dtype: str, op: str | None = None) -> np.ndarray:
    """|got - round(ref)| in ulps of the I/O dtype at max(|ref|, floor): the cancellation
    floor for LayerNorm ops, the format's own grid for every other op."""
    ref_r = oracle.round_to(ref64, dtype)
    floor = CANCEL_FLOOR[dtype] if op in CANCELLING_OPS else NATIVE_FLOOR[dtype]
    mag = np.maximum(np.abs(ref64), floor)
    ulp = np.exp2(np.floor(np.log2(mag)) - MANT_BITS[dtype])
    return np.abs(got - ref_r) / ulp


def check_y(y_gpu: torch.Tensor, y_ref: np.ndarray, what: str = "y", op: str | None = None) -> float:
    """Assert the tolerance for y of operation `op` ("ln", "rms", "fused_add_rms",
    "fused_add_ln", "softmax"); return the worst error (abs for fp32, ulps otherwise).
    Without `op` the native 16-bit grid applies (the strictest bar)."""
    dt = dtype_name(y_gpu)
    got = y_gpu.detach().cpu().double().numpy().reshape(y_ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    if dt == "fp32":
        err = float(np.abs(got - y_ref).max()) if got.size else 0.0
        assert err <= FP32_ABS_TOL, f"{what}: max abs error {err:.3g} > {FP32_ABS_TOL}"
        return err
    d = ulp_distance(got, y_ref, dt, op)
    err = float(d.max()) if d.size else 0.0
    assert err <= ULP_TOL, f"{what}: max ulp distance {err} > {ULP_TOL} (count {(d > ULP_TOL).sum()})"
    return err


def check_mean(mean_gpu: torch.Tensor, mean_ref: np.ndarray, rstd_ref: np.ndarray, eps: float):
    got = mean_gpu.detach().cpu().double().numpy().reshape(-1)
    var = np.maximum(1.0 / rstd_ref ** 2 - eps, 0.0)
    scale = np.maximum(np.abs(mean_ref), np.sqrt(var))
    err = np.abs(got - mean_ref)
    bad = err > STAT_REL_TOL * scale
    assert not bad.any(), f"mean: {bad.sum()} rows off, worst {float((err / np.maximum(scale, 1e-300)).max()):.3g}"


def check_rstd(rstd_gpu: torch.Tensor, rstd_ref: np.ndarray):
    got = rstd_gpu.detach().cpu().double().numpy().reshape(-1)
    rel = np.abs(got / rstd_ref - 1.0)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= STAT_REL_TOL, f"rstd: worst relative error {worst:.3g}"


def check_bits_equal(a: torch.Tensor, ref_bits: np.ndarray, what: str):
    dt = dtype_name(a)
    t = a.detach().cpu().contiguous()
    bits = t.view(torch.int32).numpy().view(np.uint32) if dt == "fp32" else t.view(torch.int16).numpy().view(np.uint16)
    bits = bits.reshape(ref_bits.shape)
    diff = bits != ref_bits
    assert not diff.any(), f"{what}: {int(diff.sum())} elements differ from the correctly rounded sum"


SOFTMAX_REL_TOL = 1e-5
SOFTMAX_ABS_FLOOR = 2.0 ** -126


def check_softmax_y(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    dt = dtype_name(y_gpu)
    if dt != "fp32":
        return check_y(y_gpu, y_ref, "softmax y", op="softmax")
    got = y_gpu.detach().cpu().double().numpy().reshape(y_ref.shape)
    assert np.all(np.isfinite(got)), "softmax y: non-finite outputs"
    err = np.abs(got - y_ref)
    bad = err > SOFTMAX_REL_TOL * np.abs(y_ref) + SOFTMAX_ABS_FLOOR
    assert not bad.any(), f"softmax y: {int(bad.sum())} elements off, worst relative {float((err / np.maximum(y_ref, 1e-300)).max()):.3g}"
    return float((err / np.maximum(y_ref, 1e-300)).max()) if err.size else 0.0


def check_rel(got_t: torch.Tensor, ref: np.ndarray, tol: float, what: str):
    got = got_t.detach().cpu().double().numpy().reshape(-1)
    rel = np.abs(got / ref - 1.0)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, f"{what}: worst relative error {worst:.3g}"


def check_equal_values(got_t: torch.Tensor, ref: np.ndarray, what: str):
    got = got_t.detach().cpu().double().numpy().reshape(-1)
    diff = got != ref.reshape(-1)
    assert not diff.any(), f"{what}: {int(diff.sum())} values differ"


U32 = 2.0 ** -24


def check_dx(dx_gpu: torch.Tensor, dx_ref: np.ndarray, row_scale: np.ndarray, what: str = "dx"):
    """Backward dx. row_scale S_r = rstd_r * max_j |g_j| * max(1, max_j |xhat_j|)^2 bounds
    the magnitude of every term of dx_j = rstd * (g_j - mean(g) - xhat_j * mean(g xhat)).
    An fp32 evaluation (row sums of at most 16 terms per lane, a 6-level lane tree and 16
    waves, then three roundings per element) errs by at most about 64 * 2^-24 * S_r; the
    16-bit outputs add their own rounding (1 ulp of the result)."""
    dt = dtype_name(dx_gpu)
    got = dx_gpu.detach().cpu().double().numpy().reshape(dx_ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    tol = 64 * U32 * row_scale[:, None]
    if dt != "fp32":
        mag = np.maximum(np.abs(dx_ref), GRID_FLOOR[dt])
        tol = tol + np.exp2(np.floor(np.log2(mag)) - MANT_BITS[dt])
    err = np.abs(got - dx_ref)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, worst err/tol {float((err / tol).max()):.3g}"
    return float((err / tol).max())


def check_colsum(got_t: torch.Tensor, ref: np.ndarray, abs_sum: np.ndarray, depth: float, what: str):
    """Column sums over rows (dgamma, dbeta): a sum of terms t_r whose fp32 evaluation
    passes through at most `depth` sequential additions errs by at most about
    (depth + 3) * 2^-24 * sum_r |t_r| (abs_sum); 16-bit outputs add 1 ulp of the result."""
    dt = dtype_name(got_t)
    got = got_t.detach().cpu().double().numpy().reshape(-1)
    tol = (depth + 3) * U32 * abs_sum
    if dt != "fp32":
        mag = np.maximum(np.abs(ref), GRID_FLOOR[dt])
        tol = tol + np.exp2(np.floor(np.log2(mag)) - MANT_BITS[dt])
    tol = np.maximum(tol, 1e-30)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} columns off, worst err/tol {float((err / tol).max()):.3g}"
    return float((err / tol).max())
