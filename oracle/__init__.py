"""fp64 CPU oracle for row-wise LayerNorm, RMSNorm, fused residual-add + RMSNorm /
+ LayerNorm, softmax, and the LayerNorm / RMSNorm backward passes.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package. It shares no code with the HIP library:
the arithmetic lives in ``rownorm_oracle.c`` (plain C, IEEE double), built by
``oracle/build.py`` with gcc into ``liboracle.so`` and called here through ctypes.

Functions take CPU torch tensors (or numpy arrays) holding the I/O dtype's bits and
return float64 numpy arrays. ``encode`` rounds float64 values to the I/O dtype
(round-to-nearest-even) with the oracle's own codec.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}
_TORCH_TO_NAME = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}
_BITS_NP = {"fp32": np.uint32, "fp16": np.uint16, "bf16": np.uint16}

_lib = None


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.orc_decode.argtypes = [ci, ctypes.c_uint32]
    lib.orc_decode.restype = dbl
    lib.orc_encode.argtypes = [ci, dbl]
    lib.orc_encode.restype = ctypes.c_uint32
    lib.orc_decode_array.argtypes = [ci, vp, vp, i64]
    lib.orc_decode_array.restype = None
    lib.orc_encode_array.argtypes = [ci, vp, vp, i64]
    lib.orc_encode_array.restype = None
    lib.orc_twopass_var.argtypes = [vp, i64, vp]
    lib.orc_twopass_var.restype = dbl
    lib.orc_welford_var.argtypes = [vp, i64, vp]
    lib.orc_welford_var.restype = dbl
    lib.orc_layer_norm.argtypes = [ci, vp, vp, vp, i64, i64, dbl, vp, vp, vp, ci]
    lib.orc_layer_norm.restype = ci
    lib.orc_rms_norm.argtypes = [ci, vp, vp, i64, i64, dbl, vp, vp, ci]
    lib.orc_rms_norm.restype = ci
    lib.orc_fused_add_rms_norm.argtypes = [ci, vp, vp, vp, i64, i64, dbl, vp, vp, vp, ci]
    lib.orc_fused_add_rms_norm.restype = ci
    lib.orc_fused_add_layer_norm.argtypes = [ci, vp, vp, vp, vp, i64, i64, dbl, vp, vp, vp, vp, ci]
    lib.orc_fused_add_layer_norm.restype = ci
    lib.orc_softmax.argtypes = [ci, vp, i64, i64, vp, vp, vp, ci]
    lib.orc_softmax.restype = ci
    lib.orc_layer_norm_row_f64.argtypes = [vp, vp, vp, i64, dbl, vp]
    lib.orc_layer_norm_row_f64.restype = ci
    lib.orc_rms_norm_row_f64.argtypes = [vp, vp, i64, dbl, vp]
    lib.orc_rms_norm_row_f64.restype = ci
    lib.orc_layer_norm_backward.argtypes = [ci, vp, vp, vp, vp, vp, i64, i64, dbl, vp, vp, vp]
    lib.orc_layer_norm_backward.restype = ci
    lib.orc_rms_norm_backward.argtypes = [ci, vp, vp, vp, vp, i64, i64, dbl, vp, vp]
    lib.orc_rms_norm_backward.restype = ci
    _lib = lib
    return lib


def _bits(t, dtype: str) -> np.ndarray:
    """Contiguous numpy view of the raw bits of a CPU tensor / array in ``dtype``."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if _TORCH_TO_NAME[t.dtype] != dtype:
            raise TypeError(f"tensor dtype {t.dtype} does not match {dtype}")
        if dtype == "fp32":
            return t.view(torch.int32).numpy().view(np.uint32)
        return t.view(torch.int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32 and dtype == "fp32":
        return a.view(np.uint32)
    if a.dtype == np.float16 and dtype == "fp16":
        return a.view(np.uint16)
    if a.dtype == _BITS_NP[dtype]:
        return a
    raise TypeError(f"array dtype {a.dtype} does not match {dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _check(st: int, what: str):
    if st == 1:
        raise OracleError(f"{what}: invalid arguments")
    if st == 2:
        raise OracleError(f"{what}: two-pass and Welford variances disagree")
    if st == 3:
        raise OracleError(f"{what}: out of memory")
    if st == 4:
        raise OracleError(f"{what}: plain and online softmax denominators disagree")
    if st != 0:
        raise OracleError(f"{what}: status {st}")


def dtype_name(t) -> str:
    return _TORCH_TO_NAME[t.dtype]


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of raw ``dtype`` bit patterns."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=_BITS_NP[dtype])
    out = np.empty(b.shape, dtype=np.float64)
    lib.orc_decode_array(DTYPE_CODE[dtype], _ptr(b), _ptr(out), b.size)
    return out


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (nearest, ties to even); returns raw bits."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=_BITS_NP[dtype])
    lib.orc_encode_array(DTYPE_CODE[dtype], _ptr(v), _ptr(out), v.size)
    return out


def round_to(values: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of ``values`` rounded once to ``dtype``."""
    return decode(encode(values, dtype), dtype)


def twopass_var(x: np.ndarray):
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    m = np.zeros(1)
    v = lib.orc_twopass_var(_ptr(a), a.size, _ptr(m))
    return float(m[0]), v


def welford_var(x: np.ndarray):
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    m = np.zeros(1)
    v = lib.orc_welford_var(_ptr(a), a.size, _ptr(m))
    return float(m[0]), v


def layer_norm(x, gamma=None, beta=None, eps: float = 1e-5, threads: int = 1,
               want_y: bool = True) -> Dict[str, np.ndarray]:
    """LayerNorm forward; returns {"y": [rows, N], "mean": [rows], "rstd": [rows]} in fp64."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb = _bits(x, dt)
    gb = None if gamma is None else _bits(gamma, dt)
    bb = None if beta is None else _bits(beta, dt)
    y = np.empty((rows, N), dtype=np.float64) if want_y else None
    mean = np.empty(rows, dtype=np.float64)
    rstd = np.empty(rows, dtype=np.float64)
    st = _load().orc_layer_norm(DTYPE_CODE[dt], _ptr(xb), _ptr(gb), _ptr(bb), rows, N, float(eps),
                                _ptr(y), _ptr(mean), _ptr(rstd), int(threads))
    _check(st, "layer_norm")
    return {"y": y, "mean": mean, "rstd": rstd}


def rms_norm(x, weight=None, eps: float = 1e-6, threads: int = 1, want_y: bool = True) -> Dict[str, np.ndarray]:
    """RMSNorm forward; returns {"y": [rows, N], "rstd": [rows]} in fp64."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb = _bits(x, dt)
    wb = None if weight is None else _bits(weight, dt)
    y = np.empty((rows, N), dtype=np.float64) if want_y else None
    rstd = np.empty(rows, dtype=np.float64)
    st = _load().orc_rms_norm(DTYPE_CODE[dt], _ptr(xb), _ptr(wb), rows, N, float(eps), _ptr(y), _ptr(rstd),
                              int(threads))
    _check(st, "rms_norm")
    return {"y": y, "rstd": rstd}


def fused_add_rms_norm(x, residual, weight=None, eps: float = 1e-6, threads: int = 1,
                       want_y: bool = True) -> Dict[str, np.ndarray]:
    """Fused residual add + RMSNorm; returns {"y" fp64, "residual_out" raw dtype bits, "rstd" fp64}."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb = _bits(x, dt)
    rb = _bits(residual, dt)
    wb = None if weight is None else _bits(weight, dt)
    y = np.empty((rows, N), dtype=np.float64) if want_y else None
    ro = np.empty((rows, N), dtype=_BITS_NP[dt])
    rstd = np.empty(rows, dtype=np.float64)
    st = _load().orc_fused_add_rms_norm(DTYPE_CODE[dt], _ptr(xb), _ptr(rb), _ptr(wb), rows, N, float(eps),
                                        _ptr(y), _ptr(ro), _ptr(rstd), int(threads))
    _check(st, "fused_add_rms_norm")
    return {"y": y, "residual_out": ro, "rstd": rstd}


def fused_add_layer_norm(x, residual, gamma=None, beta=None, eps: float = 1e-5, threads: int = 1,
                         want_y: bool = True) -> Dict[str, np.ndarray]:
    """Fused residual add + LayerNorm; returns {"y", "mean", "rstd"} in fp64 and
    "residual_out" as raw dtype bits."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb = _bits(x, dt)
    rb = _bits(residual, dt)
    gb = None if gamma is None else _bits(gamma, dt)
    bb = None if beta is None else _bits(beta, dt)
    y = np.empty((rows, N), dtype=np.float64) if want_y else None
    ro = np.empty((rows, N), dtype=_BITS_NP[dt])
    mean = np.empty(rows, dtype=np.float64)
    rstd = np.empty(rows, dtype=np.float64)
    st = _load().orc_fused_add_layer_norm(DTYPE_CODE[dt], _ptr(xb), _ptr(rb), _ptr(gb), _ptr(bb), rows, N,
                                          float(eps), _ptr(y), _ptr(ro), _ptr(mean), _ptr(rstd), int(threads))
    _check(st, "fused_add_layer_norm")
    return {"y": y, "residual_out": ro, "mean": mean, "rstd": rstd}


def softmax(x, threads: int = 1, want_y: bool = True) -> Dict[str, np.ndarray]:
    """Row-wise softmax; returns {"y" [rows, N], "max" [rows], "sum" [rows]} in fp64, where
    sum is the row's sum of exp(x - max)."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb = _bits(x, dt)
    y = np.empty((rows, N), dtype=np.float64) if want_y else None
    mx = np.empty(rows, dtype=np.float64)
    sm = np.empty(rows, dtype=np.float64)
    st = _load().orc_softmax(DTYPE_CODE[dt], _ptr(xb), rows, N, _ptr(y), _ptr(mx), _ptr(sm), int(threads))
    _check(st, "softmax")
    return {"y": y, "max": mx, "sum": sm}


def layer_norm_row_f64(x: np.ndarray, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm forward of one fp64 row (for derivative checks)."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float64)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=np.float64)
    y = np.empty_like(a)
    _check(_load().orc_layer_norm_row_f64(_ptr(a), _ptr(g), _ptr(b), a.size, float(eps), _ptr(y)), "ln row")
    return y


def rms_norm_row_f64(x: np.ndarray, weight=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm forward of one fp64 row (for derivative checks)."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float64)
    y = np.empty_like(a)
    _check(_load().orc_rms_norm_row_f64(_ptr(a), _ptr(w), a.size, float(eps), _ptr(y)), "rms row")
    return y


def _stats_f32(a):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().contiguous().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("statistics must be float32")
    return a


def layer_norm_backward(dy, x, gamma=None, mean=None, rstd=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """LayerNorm backward; mean / rstd (float32 [rows]) are the forward's statistics, used
    exactly as given (both None: recomputed in fp64). Returns fp64 {"dx", "dgamma", "dbeta"}."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb, db = _bits(x, dt), _bits(dy, dt)
    gb = None if gamma is None else _bits(gamma, dt)
    m, r = _stats_f32(mean), _stats_f32(rstd)
    dx = np.empty((rows, N), dtype=np.float64)
    dg = np.empty(N, dtype=np.float64)
    dbeta = np.empty(N, dtype=np.float64)
    st = _load().orc_layer_norm_backward(DTYPE_CODE[dt], _ptr(db), _ptr(xb), _ptr(gb), _ptr(m), _ptr(r), rows, N,
                                         float(eps), _ptr(dx), _ptr(dg), _ptr(dbeta))
    _check(st, "layer_norm_backward")
    return {"dx": dx, "dgamma": dg, "dbeta": dbeta}


def rms_norm_backward(dy, x, weight=None, rstd=None, eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """RMSNorm backward; rstd (float32 [rows]) from the forward, used exactly (None:
    recomputed in fp64). Returns fp64 {"dx", "dweight"}."""
    dt = dtype_name(x)
    rows, N = x.reshape(-1, x.shape[-1]).shape
    xb, db = _bits(x, dt), _bits(dy, dt)
    wb = None if weight is None else _bits(weight, dt)
    r = _stats_f32(rstd)
    dx = np.empty((rows, N), dtype=np.float64)
    dw = np.empty(N, dtype=np.float64)
    st = _load().orc_rms_norm_backward(DTYPE_CODE[dt], _ptr(db), _ptr(xb), _ptr(wb), _ptr(r), rows, N, float(eps),
                                       _ptr(dx), _ptr(dw))
    _check(st, "rms_norm_backward")
    return {"dx": dx, "dweight": dw}
