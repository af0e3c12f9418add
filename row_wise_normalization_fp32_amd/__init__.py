"""Row-wise normalization on MI355X (gfx950): LayerNorm, RMSNorm, fused residual-add +
RMSNorm / + LayerNorm, and softmax.

A thin binding over the C ABI of ``librownorm.so`` (declared in ``include/rownorm.h``):
it checks devices, layouts and dtypes, allocates outputs with torch, and passes device
pointers, row strides and torch's current HIP stream. Every step of the computation runs
in the HIP kernels of the library; there is no other implementation behind these
functions. If the library is missing, importing this package raises ``ImportError``: build
it with ``python row_wise_normalization_fp32_amd/build.py``.

Function names follow the C ABI: ``ln_forward``, ``rms_norm``, ``fused_add_rms_norm``,
``fused_add_layer_norm``, ``softmax_forward``. Inputs of shape [..., N] are treated as
[rows, N] with rows the product of the leading dimensions; they must be contiguous, except
that a 2-D tensor may have a row stride larger than N (e.g. a column slice of a wider
buffer), which the kernels read and write in place.

Every forward function also takes ``tuning=``, a dict of the fields of ``rn_tuning``
(waves_per_row, chunks_per_lane, persistent, prefetch, grid_blocks), to launch a
caller-chosen plan instead of the automatic one: for autotuning, and for measuring the
planner's choices against their alternatives.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple, Union

import torch

__all__ = [
    "ln_forward", "layer_norm", "rms_norm", "fused_add_rms_norm", "fused_add_layer_norm", "softmax_forward", "ln_backward",
    "rms_norm_backward", "backward_workspace_bytes", "forward_workspace_bytes", "plan", "plan_backward",
    "RowNormError", "LIB_PATH", "VARIANTS", "STATUS", "version",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librownorm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python row_wise_normalization_fp32_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _f32, _ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int


class RowStrides(ctypes.Structure):
    _fields_ = [("x", _i64), ("residual", _i64), ("y", _i64), ("residual_out", _i64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", _ci), ("waves_per_row", _ci), ("rows_per_block", _ci), ("block_threads", _ci),
                ("chunks_per_lane", _ci), ("grid_blocks", _i64), ("exact", _ci), ("persistent", _ci),
                ("lds_bytes", _ci), ("pairs", _ci), ("ragged", _ci)]


class Tuning(ctypes.Structure):
    _fields_ = [("waves_per_row", _ci), ("chunks_per_lane", _ci), ("persistent", _ci), ("prefetch", _ci),
                ("grid_blocks", _i64)]


_lib.rn_forward_tuned.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci,
                                  ctypes.POINTER(RowStrides), _ci, ctypes.POINTER(Tuning), _vp, ctypes.c_size_t, _vp]
_lib.rn_forward_tuned.restype = _ci
_lib.rn_plan_tuned.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _ci,
                               ctypes.POINTER(RowStrides), ctypes.POINTER(Tuning), _vp, ctypes.c_size_t,
                               ctypes.POINTER(PlanInfo)]
_lib.rn_plan_tuned.restype = _ci
_lib.rn_forward_ex.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci,
                               ctypes.POINTER(RowStrides), _ci, _vp, ctypes.c_size_t, _vp]
_lib.rn_forward_ex.restype = _ci
_lib.ln_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.ln_forward.restype = _ci
_lib.rms_norm.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.rms_norm.restype = _ci
_lib.fused_add_rms_norm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.fused_add_rms_norm.restype = _ci
_lib.fused_add_layer_norm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp]
_lib.fused_add_layer_norm.restype = _ci
_lib.softmax_forward.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _ci, _vp]
_lib.softmax_forward.restype = _ci
_lib.ln_forward_variant.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp, _ci]
_lib.ln_forward_variant.restype = _ci
_lib.rms_norm_variant.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp, _ci]
_lib.rms_norm_variant.restype = _ci
_lib.fused_add_rms_norm_variant.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _vp, _ci]
_lib.fused_add_rms_norm_variant.restype = _ci
_lib.rn_status_string.argtypes = [_ci]
_lib.rn_status_string.restype = ctypes.c_char_p
_lib.rn_version.argtypes = []
_lib.rn_version.restype = _ci
_lib.rn_plan.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci, _ci,
                         ctypes.POINTER(RowStrides), _vp, ctypes.c_size_t, ctypes.POINTER(PlanInfo)]
_lib.rn_forward_noalloc.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _ci,
                                    ctypes.POINTER(RowStrides), _vp]
_lib.rn_forward_noalloc.restype = _ci
_lib.rn_forward_workspace_bytes.argtypes = [_ci, _i64, _i64, _ci]
_lib.rn_forward_workspace_bytes.restype = ctypes.c_size_t
_lib.rn_plan.restype = _ci
_lib.rn_backward_workspace_bytes.argtypes = [_ci, _i64, _i64]
_lib.rn_backward_workspace_bytes.restype = ctypes.c_size_t
_lib.ln_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _ci, _vp, ctypes.c_size_t, _vp]
_lib.ln_backward.restype = _ci
_lib.rms_norm_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _ci, _vp, ctypes.c_size_t, _vp]
_lib.rms_norm_backward.restype = _ci
_lib.rn_plan_backward.argtypes = [_ci, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _ci, _vp, ctypes.c_size_t,
                                  ctypes.POINTER(PlanInfo)]
_lib.rn_plan_backward.restype = _ci

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
VARIANTS = {"auto": 0, "wave": 1, "workgroup": 2, "general": 3, "element": 4, "wide": 5, "wide_element": 6}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
OPS = {"ln": 0, "rms": 1, "fused_add_rms": 2, "fused_add_ln": 3, "softmax": 4}
STATUS = {0: "RN_OK", 1: "RN_ERR_NULL", 2: "RN_ERR_SHAPE", 3: "RN_ERR_DTYPE", 4: "RN_ERR_ALIAS",
          5: "RN_ERR_UNSUPPORTED", 6: "RN_ERR_HIP", 7: "RN_ERR_ALIGN", 8: "RN_ERR_WORKSPACE", 9: "RN_ERR_SCRATCH"}


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


def _row_stride(name: str, t: torch.Tensor) -> int:
    """Row stride (elements) of ``t`` seen as [rows, N]: N for contiguous tensors; a 2-D
    tensor with unit column stride may have a larger row stride."""
    if t.is_contiguous():
        return 0
    if t.dim() == 2 and t.stride(1) == 1 and t.stride(0) >= t.shape[1]:
        return t.stride(0)
    raise ValueError(f"{name} must be contiguous, or 2-D with unit column stride (rows may be padded)")


def _check_matrix(name: str, t: torch.Tensor, ref: torch.Tensor) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    if t.dtype != ref.dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {ref.dtype}")
    if t.shape != ref.shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
    return _row_stride(name, t)


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
    ld = _row_stride("x", x)
    N = x.shape[-1]
    rows = x.numel() // N if N > 0 else 0
    return rows, N, ld


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(x: torch.Tensor, stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:  # the current stream's handle without building a Stream object
        return _raw_stream(x.get_device())
    return torch.cuda.current_stream(x.device).cuda_stream


def _stats(name, t, x, rows, want):
    if not want:
        return None
    if t is None:
        t = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check_vector(name, t, x, torch.float32, rows)
    return t


def forward_workspace_bytes(op: str, rows: int, N: int, dtype: torch.dtype) -> int:
    """Workspace bytes the split-row path needs for this shape (0 when it does not apply)."""
    return int(_lib.rn_forward_workspace_bytes(OPS[op], rows, N, DTYPE_CODE[dtype]))


_ELEM_BYTES = {torch.float32: 4, torch.float16: 2, torch.bfloat16: 2}
_NO_STRIDES = RowStrides(0, 0, 0, 0)


_TUNING_DEFAULTS = {"waves_per_row": 0, "chunks_per_lane": 0, "persistent": -1, "prefetch": -1, "grid_blocks": 0}


def _tuning(tuning: Optional[dict]):
    """An rn_tuning from a dict of its fields (missing fields: automatic)."""
    if tuning is None:
        return None
    bad = set(tuning) - set(_TUNING_DEFAULTS)
    if bad:
        raise ValueError(f"unknown tuning fields {sorted(bad)}; known: {sorted(_TUNING_DEFAULTS)}")
    f = dict(_TUNING_DEFAULTS)
    f.update({k: int(v) for k, v in tuning.items()})
    return Tuning(**f)


def _call(op: str, what: str, x, residual, gamma, beta, y, ro, mean, rstd, rows, N, eps, strides, variant, stream,
          workspace=None, tuning=None):
    # Host time per call matters for small launches: the common case (dense rows, current
    # device, no workspace) takes no context manager and builds no ctypes structure.
    st_obj = _NO_STRIDES if not any(strides) else RowStrides(*strides)
    v = _variant(variant)
    ws_bytes = 0
    nb = N * _ELEM_BYTES[x.dtype]
    # only split rows use a workspace: the automatic plan splits rows beyond a workgroup's
    # registers (rows of whole 16-byte chunks up to 64 KiB, and any rows up to 16384
    # elements, never split), a forced split-row variant any rows of more than 16384 elements
    if N > 16384 and workspace is None:
        split = v in (VARIANTS["wide"], VARIANTS["wide_element"]) or (
            v == VARIANTS["auto"] and (nb > 65536 or nb % 16 != 0))
        need = forward_workspace_bytes(op, rows, N, x.dtype) if split else 0
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    head = (OPS[op], _ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(ro), _ptr(mean), _ptr(rstd),
            rows, N, float(eps), DTYPE_CODE[x.dtype], ctypes.byref(st_obj), v)
    if tuning is None:
        fn, args = _lib.rn_forward_ex, head + (_ptr(workspace), ws_bytes)
    else:
        fn, args = _lib.rn_forward_tuned, head + (ctypes.byref(_tuning(tuning)), _ptr(workspace), ws_bytes)
    if x.get_device() == torch.cuda.current_device():
        st = fn(*args, _stream(x, stream))
    else:
        with torch.cuda.device(x.device):
            st = fn(*args, _stream(x, stream))
    if st != 0:
        raise RowNormError(st, what)


def _new_like(x: torch.Tensor) -> torch.Tensor:
    return torch.empty(x.shape, dtype=x.dtype, device=x.device)


def ln_forward(x: torch.Tensor, gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
               eps: float = 1e-5, *, out: Optional[torch.Tensor] = None, mean: Optional[torch.Tensor] = None,
               rstd: Optional[torch.Tensor] = None, return_stats: bool = False, variant: Union[str, int] = "auto",
               stream=None, tuning: Optional[dict] = None):
    """LayerNorm forward over the last dimension.

    Returns ``y`` (same shape and dtype as ``x``), or ``(y, mean, rstd)`` with fp32
    per-row statistics when ``return_stats`` is true or ``mean`` / ``rstd`` are given.
    ``out`` may be ``x`` itself (in place).
    """
    rows, N, ldx = _prep(x)
    _check_vector("gamma", gamma, x)
    _check_vector("beta", beta, x)
    y = _new_like(x) if out is None else out
    ldy = _check_matrix("out", y, x)
    want = return_stats or mean is not None or rstd is not None
    mean = _stats("mean", mean, x, rows, want)
    rstd = _stats("rstd", rstd, x, rows, want)
    _call("ln", "ln_forward", x, None, gamma, beta, y, None, mean, rstd, rows, N, eps, (ldx, 0, ldy, 0), variant,
          stream, tuning=tuning)
    return (y, mean, rstd) if want else y


# The same function under the name of the usual Python wrapper of a LayerNorm kernel.
layer_norm = ln_forward


def rms_norm(x: torch.Tensor, weight: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
             out: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None, return_rstd: bool = False,
             variant: Union[str, int] = "auto", stream=None, tuning: Optional[dict] = None):
    """RMSNorm forward over the last dimension. Returns ``y`` or ``(y, rstd)``."""
    rows, N, ldx = _prep(x)
    _check_vector("weight", weight, x)
    y = _new_like(x) if out is None else out
    ldy = _check_matrix("out", y, x)
    want = return_rstd or rstd is not None
    rstd = _stats("rstd", rstd, x, rows, want)
    _call("rms", "rms_norm", x, None, weight, None, y, None, None, rstd, rows, N, eps, (ldx, 0, ldy, 0), variant,
          stream, tuning=tuning)
    return (y, rstd) if want else y


def fused_add_rms_norm(x: torch.Tensor, residual: torch.Tensor, weight: Optional[torch.Tensor] = None,
                       eps: float = 1e-6, *, out: Optional[torch.Tensor] = None,
                       residual_out: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None,
                       return_rstd: bool = False, variant: Union[str, int] = "auto", stream=None,
                       tuning: Optional[dict] = None):
    """Fused residual add + RMSNorm.

    ``residual_out = x + residual`` rounded to the dtype; ``y = rms_norm(residual_out) *
    weight``. Returns ``(y, residual_out)`` or ``(y, residual_out, rstd)``.
    """
    rows, N, ldx = _prep(x)
    ldr = _check_matrix("residual", residual, x)
    _check_vector("weight", weight, x)
    y = _new_like(x) if out is None else out
    ro = _new_like(x) if residual_out is None else residual_out
    ldy = _check_matrix("out", y, x)
    ldo = _check_matrix("residual_out", ro, x)
    want = return_rstd or rstd is not None
    rstd = _stats("rstd", rstd, x, rows, want)
    _call("fused_add_rms", "fused_add_rms_norm", x, residual, weight, None, y, ro, None, rstd, rows, N, eps,
          (ldx, ldr, ldy, ldo), variant, stream, tuning=tuning)
    return (y, ro, rstd) if want else (y, ro)


def fused_add_layer_norm(x: torch.Tensor, residual: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                         beta: Optional[torch.Tensor] = None, eps: float = 1e-5, *, out: Optional[torch.Tensor] = None,
                         residual_out: Optional[torch.Tensor] = None, mean: Optional[torch.Tensor] = None,
                         rstd: Optional[torch.Tensor] = None, return_stats: bool = False,
                         variant: Union[str, int] = "auto", stream=None, tuning: Optional[dict] = None):
    """Fused residual add + LayerNorm.

    ``residual_out = x + residual`` rounded to the dtype; ``y = layer_norm(residual_out)``.
    Returns ``(y, residual_out)`` or ``(y, residual_out, mean, rstd)``.
    """
    rows, N, ldx = _prep(x)
    ldr = _check_matrix("residual", residual, x)
    _check_vector("gamma", gamma, x)
    _check_vector("beta", beta, x)
    y = _new_like(x) if out is None else out
    ro = _new_like(x) if residual_out is None else residual_out
    ldy = _check_matrix("out", y, x)
    ldo = _check_matrix("residual_out", ro, x)
    want = return_stats or mean is not None or rstd is not None
    mean = _stats("mean", mean, x, rows, want)
    rstd = _stats("rstd", rstd, x, rows, want)
    _call("fused_add_ln", "fused_add_layer_norm", x, residual, gamma, beta, y, ro, mean, rstd, rows, N, eps,
          (ldx, ldr, ldy, ldo), variant, stream, tuning=tuning)
    return (y, ro, mean, rstd) if want else (y, ro)


def softmax_forward(x: torch.Tensor, *, out: Optional[torch.Tensor] = None, row_max: Optional[torch.Tensor] = None,
                    row_sum: Optional[torch.Tensor] = None, return_stats: bool = False,
                    variant: Union[str, int] = "auto", stream=None, tuning: Optional[dict] = None):
    """Softmax over the last dimension. Returns ``y``, or ``(y, row_max, row_sum)`` with
    row_sum = sum(exp(x - row_max)) (fp32)."""
    rows, N, ldx = _prep(x)
    y = _new_like(x) if out is None else out
    ldy = _check_matrix("out", y, x)
    want = return_stats or row_max is not None or row_sum is not None
    row_max = _stats("row_max", row_max, x, rows, want)
    row_sum = _stats("row_sum", row_sum, x, rows, want)
    _call("softmax", "softmax_forward", x, None, None, None, y, None, row_max, row_sum, rows, N, 0.0,
          (ldx, 0, ldy, 0), variant, stream, tuning=tuning)
    return (y, row_max, row_sum) if want else y


# Backward rows longer than this many elements are split across workgroups, which keep
# per-segment records in the workspace: such calls need it even without parameter gradients.
BWD_ROW_CAP = 16384


def backward_workspace_bytes(op: str, rows: int, N: int) -> int:
    """Workspace bytes a backward call with parameter gradients (or with rows longer than
    BWD_ROW_CAP elements) needs (op "ln" or "rms")."""
    return int(_lib.rn_backward_workspace_bytes(OPS[op], rows, N))


def _bwd_prep(dy, x):
    rows, N, ld = _prep(x)
    if ld != 0:
        raise ValueError("x must be contiguous for the backward pass")
    _check_matrix("dy", dy, x)
    if not dy.is_contiguous():
        raise ValueError("dy must be contiguous")
    return rows, N


def _workspace(x, op, rows, N, workspace):
    need = backward_workspace_bytes(op, rows, N)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of x")
    return workspace, workspace.numel() * workspace.element_size()


def ln_backward(dy: torch.Tensor, x: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor,
                gamma: Optional[torch.Tensor] = None, *, dx: Optional[torch.Tensor] = None, want_dx: bool = True,
                want_dgamma: bool = True, want_dbeta: bool = True, workspace: Optional[torch.Tensor] = None,
                stream=None):
    """LayerNorm backward from the forward's fp32 mean / rstd. Returns (dx, dgamma, dbeta);
    entries not wanted are None. ``dx`` may be ``dy`` or ``x`` (in place). The workspace is
    allocated with torch when not given."""
    rows, N = _bwd_prep(dy, x)
    _check_vector("gamma", gamma, x)
    _check_vector("mean", mean, x, torch.float32, rows)
    _check_vector("rstd", rstd, x, torch.float32, rows)
    if want_dx:
        dx = _new_like(x) if dx is None else dx
        _check_matrix("dx", dx, x)
        if not dx.is_contiguous():
            raise ValueError("dx must be contiguous")
    else:
        dx = None
    dg = torch.empty(N, dtype=x.dtype, device=x.device) if want_dgamma else None
    db = torch.empty(N, dtype=x.dtype, device=x.device) if want_dbeta else None
    ws, ws_bytes = (None, 0)
    if want_dgamma or want_dbeta or N > BWD_ROW_CAP:
        ws, ws_bytes = _workspace(x, "ln", rows, N, workspace)
    with torch.cuda.device(x.device):
        st = _lib.ln_backward(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dg), _ptr(db),
                              rows, N, DTYPE_CODE[x.dtype], _ptr(ws), ws_bytes, _stream(x, stream))
    if st != 0:
        raise RowNormError(st, "ln_backward")
    return dx, dg, db


def rms_norm_backward(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor, weight: Optional[torch.Tensor] = None,
                      *, dx: Optional[torch.Tensor] = None, want_dx: bool = True, want_dweight: bool = True,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """RMSNorm backward from the forward's fp32 rstd. Returns (dx, dweight)."""
    rows, N = _bwd_prep(dy, x)
    _check_vector("weight", weight, x)
    _check_vector("rstd", rstd, x, torch.float32, rows)
    if want_dx:
        dx = _new_like(x) if dx is None else dx
        _check_matrix("dx", dx, x)
        if not dx.is_contiguous():
            raise ValueError("dx must be contiguous")
    else:
        dx = None
    dw = torch.empty(N, dtype=x.dtype, device=x.device) if want_dweight else None
    ws, ws_bytes = (None, 0)
    if want_dweight or N > BWD_ROW_CAP:
        ws, ws_bytes = _workspace(x, "rms", rows, N, workspace)
    with torch.cuda.device(x.device):
        st = _lib.rms_norm_backward(_ptr(dy), _ptr(x), _ptr(weight), _ptr(rstd), _ptr(dx), _ptr(dw), rows, N,
                                    DTYPE_CODE[x.dtype], _ptr(ws), ws_bytes, _stream(x, stream))
    if st != 0:
        raise RowNormError(st, "rms_norm_backward")
    return dx, dw


def plan_backward(op: str, rows: int, N: int, dtype: torch.dtype, *, ptrs: Optional[dict] = None,
                  workspace_bytes: Optional[int] = None) -> Tuple[int, dict]:
    """Host-only backward plan. ``ptrs`` maps dy, x, gamma, mean, rstd, dx, dgamma, dbeta,
    workspace to addresses (defaults: non-overlapping, aligned; dgamma / dbeta / workspace
    absent unless given)."""
    s = torch.tensor([], dtype=dtype).element_size() if isinstance(dtype, torch.dtype) else 4
    step = ((max(1, rows * N * s) + 4095) // 4096 + 1) * 4096
    base = 1 << 40
    p = {"dy": base, "x": base + step, "dx": base + 2 * step, "mean": base + 3 * step,
         "rstd": base + 3 * step + ((rows * 4 + 4095) // 4096 + 1) * 4096}
    if ptrs:
        p.update(ptrs)
    wsb = backward_workspace_bytes(op, rows, N) if workspace_bytes is None else workspace_bytes
    info = PlanInfo()
    st = _lib.rn_plan_backward(OPS[op], p.get("dy"), p.get("x"), p.get("gamma"), p.get("mean"), p.get("rstd"),
                               p.get("dx"), p.get("dgamma"), p.get("dbeta"), rows, N, DTYPE_CODE.get(dtype, 99),
                               p.get("workspace"), wsb, ctypes.byref(info))
    return st, {"variant": VARIANT_NAMES.get(info.variant, info.variant), "waves_per_row": info.waves_per_row,
                "rows_per_block": info.rows_per_block, "block_threads": info.block_threads,
                "chunks_per_lane": info.chunks_per_lane, "grid_blocks": info.grid_blocks,
                "exact": bool(info.exact), "lds_bytes": info.lds_bytes,
                "pairs": bool(info.pairs)}


def plan(op: str, rows: int, N: int, dtype: torch.dtype, *, ptrs: Optional[dict] = None, eps: float = 1e-5,
         variant: Union[str, int] = "auto", strides: Optional[dict] = None,
         workspace_bytes: int = 0, tuning: Optional[dict] = None) -> Tuple[int, dict]:
    """Host-only launch plan (no GPU needed). ``ptrs`` maps buffer names (x, residual,
    gamma, beta, y, residual_out, mean, rstd) to integer addresses; missing required
    buffers default to 256-byte-aligned placeholders that never overlap. ``strides`` maps
    x / residual / y / residual_out to row strides in elements; ``workspace_bytes`` > 0
    stands for a workspace of that size (the split-row path); ``tuning`` (fields of
    rn_tuning) gives the plan rn_forward_tuned would launch, with status RN_ERR_UNSUPPORTED
    when no kernel of that shape is built. Returns ``(status, info)``."""
    s = torch.tensor([], dtype=dtype).element_size()
    ld = max([N] + list((strides or {}).values()))
    span = max(1, rows * ld * s)
    base = 1 << 40
    step = ((span + 4095) // 4096 + 1) * 4096
    default = {"x": base, "residual": base + step, "y": base + 2 * step, "residual_out": base + 3 * step}
    p = dict(default)
    if op not in ("fused_add_rms", "fused_add_ln"):
        p.pop("residual")
        p.pop("residual_out")
    if ptrs:
        p.update(ptrs)
    st_obj = RowStrides(**(strides or {}))
    info = PlanInfo()
    head = (OPS[op], p.get("x"), p.get("residual"), p.get("gamma"), p.get("beta"), p.get("y"), p.get("residual_out"),
            p.get("mean"), p.get("rstd"), rows, N, float(eps), DTYPE_CODE.get(dtype, 99), _variant(variant),
            ctypes.byref(st_obj))
    tail = (p.get("workspace", (1 << 47) if workspace_bytes else None), workspace_bytes, ctypes.byref(info))
    if tuning is None:
        st = _lib.rn_plan(*head, *tail)
    else:
        st = _lib.rn_plan_tuned(*head, ctypes.byref(_tuning(tuning)), *tail)
    return st, {"variant": VARIANT_NAMES.get(info.variant, info.variant), "waves_per_row": info.waves_per_row,
                "rows_per_block": info.rows_per_block, "block_threads": info.block_threads,
                "chunks_per_lane": info.chunks_per_lane, "grid_blocks": info.grid_blocks,
                "exact": bool(info.exact), "persistent": bool(info.persistent), "lds_bytes": info.lds_bytes,
                "pairs": bool(info.pairs), "ragged": bool(info.ragged)}
