"""Seeded synthetic inputs for the row-wise normalization workloads.

This module is shared by the oracle's tests, the HIP parity tests, ``smoke()`` and
``bench.py``. It draws random numbers and rounds them to the I/O dtype, nothing else:
it holds none of the normalization arithmetic, so neither side of a parity test can
borrow the other's arithmetic through it.

Recipe (the same for every workload, so a reader can regenerate any input by hand):

* ``numpy.random.Generator(numpy.random.PCG64(seed))``;
* draws in float64, in this order: the per-column parameters (gamma, then beta, or
  the RMSNorm weight), the per-row constants (offset, or mean then std), x, then the
  residual;
* each array is rounded once, round-to-nearest-even, from float64 straight to the I/O
  dtype (``round_once``: the value is scaled by a power of two so that the dtype's last
  mantissa bit has weight 1, rounded to an integer by ``numpy.rint``, and scaled back;
  every step but the ``rint`` is exact). A detour through float32 would round twice,
  and for arbitrary float64 values that differs from one rounding at a few values per
  million. The rounding of inputs is immaterial to parity: both the oracle and the GPU
  receive the identical bits.

The five headline workloads follow the shapes the pages measure: the LayerNorm
walkthrough's "mean away from 0, variance away from 1" input advice at N=1024
(LayerNorm CUDA walkthrough, lpnh.cn/news/2756757, section 2.1), the LLM-operators
lesson's LayerNorm (128 x 4096) and RMSNorm (2048 x 4096) shapes (smarter.xin
"05 LLM Ops", results tables), the fused RMSNorm article's 256 x 4096 FP16 headline
shape (diycv.top "cuda-fused-rmsnorm-kernel", section 7), and the walkthrough's
16384-wide row that no longer fits one block (section 1.1).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: an op, an I/O dtype, a shape, eps and input distributions.

    ``x_dist`` selects how x is drawn:
      * ``"normal"``     x = x_loc + x_scale * z
      * ``"row_offset"`` x = c_r + z with c_r ~ U(-row_offset, row_offset) per row
      * ``"row_mean_std"`` x = m_r + s_r * z with m_r ~ U(-mean_range, mean_range),
        s_r ~ U(std_lo, std_hi) per row
      * ``"constant"``   every row is one constant drawn ~ U(-row_offset, row_offset)
    z ~ N(0, 1) i.i.d. per element.
    """

    name: str
    op: str  # "ln", "rms", "fused_add_rms", "fused_add_ln", "softmax", "ln_bwd", "rms_bwd"
    dtype: str  # "fp32", "fp16", "bf16"
    rows: int
    N: int
    eps: float
    seed: int
    x_dist: str = "normal"
    x_loc: float = 0.0
    x_scale: float = 1.0
    row_offset: float = 0.0
    mean_range: float = 0.0
    std_lo: float = 1.0
    std_hi: float = 1.0
    residual_scale: float = 2.0
    dy_scale: float = 1.0  # backward: dy ~ N(0, dy_scale^2)
    param_lo: float = 0.5  # gamma / weight ~ U(param_lo, param_hi)
    param_hi: float = 1.5
    beta_scale: float = 0.1  # beta ~ N(0, beta_scale^2)
    with_gamma: bool = True
    with_beta: bool = True

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def scaled(self, rows: Optional[int] = None, N: Optional[int] = None, seed: Optional[int] = None,
               name: Optional[str] = None, **kw) -> "Workload":
        """A copy with another shape / seed (same distributions)."""
        return dataclasses.replace(self, rows=self.rows if rows is None else rows,
                                   N=self.N if N is None else N,
                                   seed=self.seed if seed is None else seed,
                                   name=name or self.name, **kw)


# The five configurations. Seeds: 1000 + config number; the bf16 variant of the fused
# config adds 10. "Normal(0, 2)" for the residual is read as standard deviation 2, the
# same convention as "Normal(mean=5, std=3)" for the first config.
C1 = Workload("C1_ln_fp32_64x1024", "ln", "fp32", 64, 1024, 1e-5, 1001,
              x_dist="normal", x_loc=5.0, x_scale=3.0)
C2 = Workload("C2_ln_fp32_128x4096_offset", "ln", "fp32", 128, 4096, 1e-5, 1002,
              x_dist="row_offset", row_offset=1000.0)
C3 = Workload("C3_rms_fp16_2048x4096", "rms", "fp16", 2048, 4096, 1e-6, 1003)
C4_FP16 = Workload("C4_fused_fp16_256x4096", "fused_add_rms", "fp16", 256, 4096, 1e-6, 1004,
                   residual_scale=2.0)
C4_BF16 = Workload("C4_fused_bf16_256x4096", "fused_add_rms", "bf16", 256, 4096, 1e-6, 1014,
                   residual_scale=2.0)
C5 = Workload("C5_ln_bf16_4096x16384", "ln", "bf16", 4096, 16384, 1e-5, 1005,
              x_dist="row_mean_std", mean_range=10.0, std_lo=0.5, std_hi=4.0)

CONFIGS = (C1, C2, C3, C4_FP16, C4_BF16, C5)

# Fused residual add + LayerNorm: the fused config's shape and residual, LayerNorm
# parameters and the row-wise input spread of the 16384-wide config.
FUSED_LN = Workload("fused_ln_bf16_256x4096", "fused_add_ln", "bf16", 256, 4096, 1e-5, 1021,
                    x_dist="row_mean_std", mean_range=10.0, std_lo=0.5, std_hi=4.0, residual_scale=2.0)
FUSED_LN_8192 = FUSED_LN.scaled(rows=8192, seed=1121, name="fused_ln_bf16_8192x4096")

# Softmax: the LLM-ops lesson's measured shape (batch 128 x sequence 4096, fp32 I/O) with
# logits x = 2 z, and a 32M-element version of it for bandwidth.
SOFTMAX = Workload("softmax_fp32_128x4096", "softmax", "fp32", 128, 4096, 0.0, 1031, x_scale=2.0)
SOFTMAX_8192 = SOFTMAX.scaled(rows=8192, seed=1131, name="softmax_fp32_8192x4096")

# Backward passes: LayerNorm over the 16384-wide config's rows, RMSNorm over the RMSNorm
# config's rows; dy ~ N(0, 1).
LN_BWD = Workload("ln_bwd_bf16_4096x16384", "ln_bwd", "bf16", 4096, 16384, 1e-5, 1041,
                  x_dist="row_mean_std", mean_range=10.0, std_lo=0.5, std_hi=4.0)
RMS_BWD = Workload("rms_bwd_fp16_2048x4096", "rms_bwd", "fp16", 2048, 4096, 1e-6, 1043)

# Larger fused add+RMSNorm shape with the fused config's distributions: 8192 x 4096 is
# 32M elements, past the 8M-element size where the bandwidth target applies.
FUSED_8192 = C4_FP16.scaled(rows=8192, seed=1104, name="fused_fp16_8192x4096")


# (explicit mantissa bits, exponent of the smallest normal) of each I/O dtype
_FORMAT = {"fp32": (23, -126), "fp16": (10, -14), "bf16": (7, -126)}


def round_once(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values rounded once (nearest, ties to even) to ``dtype``, still as float64.

    With |v| = m * 2^k, 0.5 <= m < 1, the dtype's spacing at v is 2^(max(k - 1, emin) - mant);
    v / spacing is exact, ``rint`` rounds it to the nearest integer (ties to even) and the
    product with the spacing is exact again. Inputs here stay far inside every format's
    range, so overflow is not handled."""
    mant, emin = _FORMAT[dtype]
    a = np.ascontiguousarray(a, dtype=np.float64)
    _, k = np.frexp(a)
    e = np.maximum(k - 1, emin) - mant
    return np.ldexp(np.rint(np.ldexp(a, -e)), e)


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    # the rounded values are exact in float32 and in the dtype: the conversions are exact
    return torch.from_numpy(round_once(a, dtype)).to(torch.float32).to(TORCH_DTYPES[dtype])


def make_inputs(w: Workload) -> Dict[str, torch.Tensor]:
    """Draw the inputs of ``w`` as CPU tensors in the I/O dtype.

    Keys: ``x`` [rows, N]; ``residual`` [rows, N] (fused ops); ``dy`` [rows, N]
    (backward ops); ``gamma`` and ``beta`` [N] (LayerNorm ops; absent when disabled) or
    ``weight`` [N] (RMSNorm ops); softmax has no parameters.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    out: Dict[str, torch.Tensor] = {}
    if w.op == "softmax":
        pass
    elif w.op in ("ln", "fused_add_ln", "ln_bwd"):
        g = rng.uniform(w.param_lo, w.param_hi, size=w.N)
        b = w.beta_scale * rng.standard_normal(size=w.N)
        if w.with_gamma:
            out["gamma"] = _to_dtype(g, w.dtype)
        if w.with_beta:
            out["beta"] = _to_dtype(b, w.dtype)
    else:
        wt = rng.uniform(w.param_lo, w.param_hi, size=w.N)
        if w.with_gamma:
            out["weight"] = _to_dtype(wt, w.dtype)

    shape = (w.rows, w.N)
    if w.x_dist == "normal":
        x = w.x_loc + w.x_scale * rng.standard_normal(size=shape)
    elif w.x_dist == "row_offset":
        c = rng.uniform(-w.row_offset, w.row_offset, size=(w.rows, 1))
        x = c + rng.standard_normal(size=shape)
    elif w.x_dist == "row_mean_std":
        m = rng.uniform(-w.mean_range, w.mean_range, size=(w.rows, 1))
        s = rng.uniform(w.std_lo, w.std_hi, size=(w.rows, 1))
        x = m + s * rng.standard_normal(size=shape)
    elif w.x_dist == "constant":
        c = rng.uniform(-w.row_offset, w.row_offset, size=(w.rows, 1))
        x = np.broadcast_to(c, shape)
    else:
        raise ValueError(f"unknown x_dist {w.x_dist!r}")
    out["x"] = _to_dtype(x, w.dtype)
    if w.op in ("fused_add_rms", "fused_add_ln"):
        out["residual"] = _to_dtype(w.residual_scale * rng.standard_normal(size=shape), w.dtype)
    if w.op in ("ln_bwd", "rms_bwd"):
        out["dy"] = _to_dtype(w.dy_scale * rng.standard_normal(size=shape), w.dtype)
    return out


def algorithmic_bytes(op: str, rows: int, N: int, elem_bytes: int, with_params: bool = True,
                      with_stats: bool = False, with_beta: bool = True) -> int:
    """Minimum HBM bytes one call must move: every tensor read once and written once.

    LayerNorm: read x, write y, read gamma and beta once (+ 8 bytes per row for fp32
    mean and rstd when requested). RMSNorm: read x, write y, read weight once (+ 4
    bytes per row for rstd). Fused add + RMSNorm: read x and residual, write y and
    residual_out, read weight once (+ 4 bytes per row for rstd). Fused add + LayerNorm:
    the same with gamma and beta (+ 8 bytes per row). Softmax: read x, write y.
    LayerNorm backward: read x, dy, gamma, mean and rstd, write dx, dgamma and dbeta;
    RMSNorm backward: read x, dy, weight and rstd, write dx and dweight.
    """
    elems = rows * N * elem_bytes
    if op == "ln":
        b = 2 * elems + (N * elem_bytes if with_params else 0) + (N * elem_bytes if with_params and with_beta else 0)
        return b + (8 * rows if with_stats else 0)
    if op == "rms":
        return 2 * elems + (N * elem_bytes if with_params else 0) + (4 * rows if with_stats else 0)
    if op == "fused_add_rms":
        return 4 * elems + (N * elem_bytes if with_params else 0) + (4 * rows if with_stats else 0)
    if op == "fused_add_ln":
        return 4 * elems + (2 * N * elem_bytes if with_params else 0) + (8 * rows if with_stats else 0)
    if op == "softmax":
        return 2 * elems
    if op == "ln_bwd":
        return 3 * elems + (3 if with_params else 2) * N * elem_bytes + 8 * rows
    if op == "rms_bwd":
        return 3 * elems + (2 if with_params else 1) * N * elem_bytes + 4 * rows
    raise ValueError(op)

# General shapes with the input distributions of the configs above: rows that are not whole
# 16-byte chunks (the 16384-wide config's distributions at N = 4095), rows beyond a
# workgroup's registers (the offset-row config at N = 65536, fp32), and a vocabulary-sized
# softmax (N = 50257 logits, fp32, not whole chunks).
LN_RAGGED = C5.scaled(rows=16384, N=4095, seed=1205, name="ln_bf16_16384x4095")
LN_SPLIT = C2.scaled(rows=1024, N=65536, seed=1202, name="ln_fp32_1024x65536")
SOFTMAX_VOCAB = SOFTMAX.scaled(rows=1024, N=50257, seed=1231, name="softmax_fp32_1024x50257")
