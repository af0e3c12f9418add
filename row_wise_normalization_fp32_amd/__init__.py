"""Row-wise normalization on MI355X (gfx950): LayerNorm, RMSNorm, fused residual-add + RMSNorm.

A thin binding over the C ABI of ``librownorm.so`` (declared in ``include/rownorm.h``):
it checks devices, contiguity and dtypes, allocates outputs with torch, and passes device
pointers and torch's current HIP stream. Every step of the computation runs in the HIP
kernels of the library; there is no other implementation behind these functions. If the
library is missing, importing this package raises ``ImportError``: build it with
``python row_wise_normalization_fp32_amd/build.py``.

Function names follow the C ABI: ``ln_forward``, ``rms_norm``, ``fused_add_rms_norm``.
Inputs of shape [..., N] are treated as [rows, N] with rows the product of the leading
dimensions.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple, Union

import torch

__all__ = [
    "ln_forward", "rms_norm", "fused_add_rms_norm", "plan", "RowNormError", "LIB_PATH",
    "VARIANTS", "STATUS", "version",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librownorm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python row_wise_normalization_fp32_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _f32, _ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
_lib.ln_forward_variant.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp, _ci]
_lib.ln_forward_variant.restype = _ci
_lib.rms_norm_variant.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp, _ci]
_lib.rms_norm_variant.restype = _ci
_lib.fused_add_rms_norm_variant.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp, _ci]
_lib.fused_add_rms_norm_variant.restype = _ci
_lib.ln_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.ln_forward.restype = _ci
_lib.rms_norm.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.rms_norm.restype = _ci
_lib.fused_add_rms_norm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.fused_add_rms_norm.restype = _ci
_lib.rn_status_string.argtypes = [_ci]
_lib.rn_status_string.restype = ctypes.c_char_p
_lib.rn_version.argtypes = []
_lib.rn_version.restype = _ci


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", _ci), ("waves_per_row", _ci), ("rows_per_block", _ci), ("block_threads", _ci),
                ("chunks_per_lane", _ci), ("grid_blocks", _i64), ("exact", _ci), ("persistent", _ci),
                ("lds_bytes", _ci)]


_lib.rn_plan.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _ci,
                         ctypes.POINTER(PlanInfo)]
_lib.rn_plan.restype = _ci

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
VARIANTS = {"auto": 0, "wave": 1, "workgroup": 2, "general": 3}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
OPS = {"ln": 0, "rms": 1, "fused_add_rms": 2}
STATUS = {0: "RN_OK", 1: "RN_ERR_NULL", 2: "RN_ERR_SHAPE", 3: "RN_ERR_DTYPE", 4: "RN_ERR_ALIAS",
          5: "RN_ERR_UNSUPPORTED", 6: "RN_ERR_HIP", 7: "RN_ERR_ALIGN"}


class RowNormError(RuntimeError):
    """Non-zero status from the C ABI; ``.status`` holds the code."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.rn_status_string(status).decode()} ({status})")


def version() -> int:
    return _lib.rn_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _variant(v: Union[str, int]) -> int:
    return VARIANTS[v] if isinstance(v, str) else int(v)


def _check_matrix(name: str, t: torch.Tensor, ref: torch.Tensor):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    if t.dtype != ref.dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {ref.dtype}")
    if t.shape != ref.shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense rows)")


def _check_vector(name: str, t: Optional[torch.Tensor], ref: torch.Tensor, dtype=None, n=None):
    if t is None:
        return
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    want = ref.dtype if dtype is None else dtype
    if t.dtype != want:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {want}")
    n = ref.shape[-1] if n is None else n
    if t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of {n} elements")


def _prep(x: torch.Tensor):
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor (HIP device)")
    if x.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {x.dtype}; use float32, float16 or bfloat16")
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (dense rows)")
    N = x.shape[-1]
    rows = x.numel() // N if N > 0 else 0
    return rows, N


def _stream(x: torch.Tensor, stream) -> int:
    s = torch.cuda.current_stream(x.device) if stream is None else stream
    return s.cuda_stream


def ln_forward(x: torch.Tensor, gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
               eps: float = 1e-5, *, out: Optional[torch.Tensor] = None, mean: Optional[torch.Tensor] = None,
               rstd: Optional[torch.Tensor] = None, return_stats: bool = False, variant: Union[str, int] = "auto",
               stream=None):
    """LayerNorm forward over the last dimension.

    Returns ``y`` (same shape and dtype as ``x``), or ``(y, mean, rstd)`` with fp32
    per-row statistics when ``return_stats`` is true or ``mean`` / ``rstd`` are given.
    ``out`` may be ``x`` itself (in place).
    """
    rows, N = _prep(x)
    _check_vector("gamma", gamma, x)
    _check_vector("beta", beta, x)
    y = torch.empty_like(x) if out is None else out
    _check_matrix("out", y, x)
    want_stats = return_stats or mean is not None or rstd is not None
    if want_stats:
        if mean is None:
            mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        if rstd is None:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        _check_vector("mean", mean, x, torch.float32, rows)
        _check_vector("rstd", rstd, x, torch.float32, rows)
    with torch.cuda.device(x.device):
        st = _lib.ln_forward_variant(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), rows, N,
                                     float(eps), DTYPE_CODE[x.dtype], _stream(x, stream), _variant(variant))
    if st != 0:
        raise RowNormError(st, "ln_forward")
    return (y, mean, rstd) if want_stats else y


def rms_norm(x: torch.Tensor, weight: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
             out: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None, return_rstd: bool = False,
             variant: Union[str, int] = "auto", stream=None):
    """RMSNorm forward over the last dimension. Returns ``y`` or ``(y, rstd)``."""
    rows, N = _prep(x)
    _check_vector("weight", weight, x)
    y = torch.empty_like(x) if out is None else out
    _check_matrix("out", y, x)
    want = return_rstd or rstd is not None
    if want:
        if rstd is None:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        _check_vector("rstd", rstd, x, torch.float32, rows)
    with torch.cuda.device(x.device):
        st = _lib.rms_norm_variant(_ptr(x), _ptr(weight), _ptr(y), _ptr(rstd), rows, N, float(eps),
                                   DTYPE_CODE[x.dtype], _stream(x, stream), _variant(variant))
    if st != 0:
        raise RowNormError(st, "rms_norm")
    return (y, rstd) if want else y


def fused_add_rms_norm(x: torch.Tensor, residual: torch.Tensor, weight: Optional[torch.Tensor] = None,
                       eps: float = 1e-6, *, out: Optional[torch.Tensor] = None,
                       residual_out: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None,
                       return_rstd: bool = False, variant: Union[str, int] = "auto", stream=None):
    """Fused residual add + RMSNorm.

    ``residual_out = x + residual`` rounded to the dtype; ``y = rms_norm(residual_out) *
    weight``. Returns ``(y, residual_out)`` or ``(y, residual_out, rstd)``.
    """
    rows, N = _prep(x)
    _check_matrix("residual", residual, x)
    _check_vector("weight", weight, x)
    y = torch.empty_like(x) if out is None else out
    ro = torch.empty_like(x) if residual_out is None else residual_out
    _check_matrix("out", y, x)
    _check_matrix("residual_out", ro, x)
    want = return_rstd or rstd is not None
    if want:
        if rstd is None:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        _check_vector("rstd", rstd, x, torch.float32, rows)
    with torch.cuda.device(x.device):
        st = _lib.fused_add_rms_norm_variant(_ptr(x), _ptr(residual), _ptr(weight), _ptr(y), _ptr(ro), _ptr(rstd),
                                             rows, N, float(eps), DTYPE_CODE[x.dtype], _stream(x, stream),
                                             _variant(variant))
    if st != 0:
        raise RowNormError(st, "fused_add_rms_norm")
    return (y, ro, rstd) if want else (y, ro)


def plan(op: str, rows: int, N: int, dtype: torch.dtype, *, ptrs: Optional[dict] = None, eps: float = 1e-5,
         variant: Union[str, int] = "auto") -> Tuple[int, dict]:
    """Host-only launch plan (no GPU needed). ``ptrs`` maps buffer names (x, residual,
    gamma, beta, y, residual_out, mean, rstd) to integer addresses; missing required
    buffers default to 256-byte-aligned placeholders that never overlap. Returns
    ``(status, info)``."""
    s = torch.tensor([], dtype=dtype).element_size()
    span = max(1, rows * N * s)
    base = 1 << 40
    step = ((span + 4095) // 4096 + 1) * 4096
    default = {"x": base, "residual": base + step, "y": base + 2 * step, "residual_out": base + 3 * step}
    p = dict(default)
    if op != "fused_add_rms":
        p.pop("residual")
        p.pop("residual_out")
    if ptrs:
        p.update(ptrs)
    info = PlanInfo()
    st = _lib.rn_plan(OPS[op], p.get("x"), p.get("residual"), p.get("gamma"), p.get("beta"), p.get("y"),
                      p.get("residual_out"), p.get("mean"), p.get("rstd"), rows, N, float(eps),
                      DTYPE_CODE.get(dtype, 99), _variant(variant), ctypes.byref(info))
    return st, {"variant": VARIANT_NAMES.get(info.variant, info.variant), "waves_per_row": info.waves_per_row,
                "rows_per_block": info.rows_per_block, "block_threads": info.block_threads,
                "chunks_per_lane": info.chunks_per_lane, "grid_blocks": info.grid_blocks,
                "exact": bool(info.exact), "persistent": bool(info.persistent), "lds_bytes": info.lds_bytes}
