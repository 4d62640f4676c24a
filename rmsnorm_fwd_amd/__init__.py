"""Python binding of the MI355X training-RMSNorm library (librmsnorm_mi355x.so).

Argument marshalling only: every step of the forward and backward runs in the
library's HIP kernels.  The functions carry the C ABI's names
(include/rmsnorm.h); they take torch tensors for device memory and use torch's
current stream, and they allocate outputs with torch when none are given.

The library must have been built (``python -m rmsnorm_fwd_amd.build`` or
``__graft_entry__.build()``); there is no fallback implementation, and a
missing library raises on first use.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm_mi355x.so")

RMSN_OK = 0
RMSN_ERR_INVALID_ARG = 1
RMSN_ERR_UNSUPPORTED = 2
RMSN_ERR_MISALIGNED = 3
RMSN_ERR_WORKSPACE = 4
RMSN_ERR_HIP = 5
RMSN_W_BF16 = 0
RMSN_W_F32 = 1
RMSN_FORM_PAIR = 0
RMSN_FORM_ATOMIC = 1
RMSN_FORM_COLS = 2
RMSN_FORM_COLS_TICKET = 3
RMSN_MAX_H = 16384
RMSN_NOALLOC_SCRATCH_BYTES = 32 << 20

# every symbol include/rmsnorm.h declares
EXPORTS = (
    "rmsnorm_fwd",
    "rmsnorm_bwd_workspace_size",
    "rmsnorm_bwd_workspace_init",
    "rmsnorm_bwd",
    "rmsnorm_bwd_route",
    "rmsnorm_gated_bwd_route",
    "rmsnorm_bwd_workspace_size_for_route",
    "rmsnorm_bwd_routed",
    "rmsnorm_gated_fwd",
    "rmsnorm_gated_bwd",
    "rmsnorm_bwd_noalloc",
    "rmsnorm_status_string",
)


class RmsnRoute(ctypes.Structure):
    """(form, chunks, col_chunks, col_vecs, prefetch); col_chunks and
    col_vecs are 0 except for the column forms, prefetch 0 or 1 (pair and
    atomic forms only).  Fields left out of a shorter tuple are 0."""
    _fields_ = [("form", ctypes.c_int32), ("chunks", ctypes.c_int32), ("col_chunks", ctypes.c_int32),
                ("col_vecs", ctypes.c_int32), ("prefetch", ctypes.c_int32)]


class RmsnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -m rmsnorm_fwd_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.rmsnorm_fwd.argtypes = [vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i64,
                              ctypes.c_double, i32, vp]
    L.rmsnorm_fwd.restype = i32
    L.rmsnorm_bwd_workspace_size.argtypes = [i64, i64, i64, i32, vp, i32]
    L.rmsnorm_bwd_workspace_size.restype = ctypes.c_size_t
    L.rmsnorm_bwd_workspace_init.argtypes = [vp, ctypes.c_size_t, i64, vp]
    L.rmsnorm_bwd_workspace_init.restype = i32
    L.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, ctypes.c_size_t,
                              i64, i64, i64, i64, i64, i32, vp]
    L.rmsnorm_bwd.restype = i32
    L.rmsnorm_bwd_route.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(RmsnRoute)]
    L.rmsnorm_gated_bwd_route.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(RmsnRoute)]
    L.rmsnorm_bwd_route.restype = i32
    L.rmsnorm_gated_bwd_route.restype = i32
    L.rmsnorm_bwd_workspace_size_for_route.argtypes = [i64, i64, i64, RmsnRoute]
    L.rmsnorm_bwd_workspace_size_for_route.restype = ctypes.c_size_t
    L.rmsnorm_bwd_routed.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, ctypes.c_size_t,
                                     i64, i64, i64, i64, i64, i32, RmsnRoute, vp]
    L.rmsnorm_bwd_routed.restype = i32
    L.rmsnorm_gated_fwd.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, i64, ctypes.c_double, i32, vp]
    L.rmsnorm_gated_fwd.restype = i32
    L.rmsnorm_gated_bwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, ctypes.c_size_t,
                                    i64, i64, i64, i64, i64, i32, vp]
    L.rmsnorm_gated_bwd.restype = i32
    L.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    L.rmsnorm_bwd_noalloc.restype = i32
    L.rmsnorm_status_string.argtypes = [i32]
    L.rmsnorm_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().rmsnorm_status_string(int(status)).decode()


def _check(fn, status):
    if status != RMSN_OK:
        raise RmsnError(fn, status)


# ------------------------------------------------------------- helpers ----

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def geometry(t):
    """(T, heads, H, stride_t, stride_h) of a [T,H] or [T,heads,H] tensor
    whose last dimension is contiguous."""
    if t.dim() == 2:
        T, H = t.shape
        if t.stride(1) != 1:
            raise ValueError("the last dimension must be contiguous")
        return T, 1, H, (t.stride(0) if T > 1 else H), H
    if t.dim() == 3:
        T, heads, H = t.shape
        if t.stride(2) != 1:
            raise ValueError("the last dimension must be contiguous")
        sh = t.stride(1) if heads > 1 else H
        st = t.stride(0) if T > 1 else heads * sh
        return T, heads, H, st, sh
    raise ValueError("expected a [T,H] or [T,heads,H] tensor")


def _same_geometry(a, b, what):
    if b is not None and (tuple(a.shape) != tuple(b.shape) or geometry(a) != geometry(b)):
        raise ValueError(f"{what} must have the shape and strides of x")


def _like(x):
    torch = _torch()
    return torch.empty_strided(x.shape, x.stride(), dtype=torch.bfloat16, device=x.device)


def _w_dtype(w):
    torch = _torch()
    if w.dtype == torch.bfloat16:
        return RMSN_W_BF16
    if w.dtype == torch.float32:
        return RMSN_W_F32
    raise TypeError("w must be bfloat16 or float32")


# The C ABI sees plain pointers: the sizes, dtypes and devices that it cannot
# check are checked here, before any call into the library.

def _device_of(t, what, device):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{what} must be a GPU tensor on {device}, got {t.device}")


def _act(t, what, x):
    """An activation tensor ([T,H] or [T,heads,H], strides checked apart): BF16, on x's device."""
    if t is None:
        return
    if t.dtype != _torch().bfloat16:
        raise TypeError(f"{what} must be bfloat16, got {t.dtype}")
    _device_of(t, what, x.device)


def _vec(t, what, n, dtypes, device):
    """A contiguous [n] vector of one of `dtypes` on `device`."""
    if t.dtype not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.dim() != 1 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous [{n}] tensor, got shape {tuple(t.shape)}")
    _device_of(t, what, device)


def _weight(w, H, device):
    torch = _torch()
    _vec(w, "w", H, (torch.bfloat16, torch.float32), device)


def _workspace(ws, device):
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _device_of(ws, "workspace", device)


# ------------------------------------------------------------ forward ----

def rmsnorm_fwd(x, w, eps: float = 1e-6, residual=None, deterministic: bool = True, *,
                y=None, residual_out=None, rstd=None, stream=None):
    """y, rstd (and h = x + residual) of the training RMSNorm forward.

    Returns (y, rstd, residual_out); residual_out is None without a residual."""
    torch = _torch()
    _act(x, "x", x)
    T, heads, H, st, sh = geometry(x)
    _act(residual, "residual", x)
    _same_geometry(x, residual, "residual")
    y = _like(x) if y is None else y
    _act(y, "y", x)
    _same_geometry(x, y, "y")
    if residual is not None and residual_out is None:
        residual_out = _like(x)
    _act(residual_out, "residual_out", x)
    _same_geometry(x, residual_out, "residual_out")
    _weight(w, H, x.device)
    if rstd is None:
        rstd = torch.empty(T * heads, dtype=torch.float32, device=x.device)
    _vec(rstd, "rstd", T * heads, (torch.float32,), x.device)
    st_ = lib().rmsnorm_fwd(_ptr(x), _ptr(residual), _ptr(w), _w_dtype(w), _ptr(y),
                            _ptr(residual_out), _ptr(rstd), T, heads, H, st, sh, float(eps),
                            int(bool(deterministic)), _stream(x.device, stream))
    _check("rmsnorm_fwd", st_)
    return y, rstd, residual_out


# ----------------------------------------------------------- backward ----

def rmsnorm_bwd_workspace_size(T: int, heads: int, H: int, w_dtype: int = RMSN_W_BF16,
                               has_residual: bool = False, deterministic: bool = True) -> int:
    """Bytes rmsnorm_bwd needs for these arguments (0 if they are invalid).
    The C call takes the dres pointer itself; only whether it is NULL counts,
    so a stand-in non-NULL address is passed for has_residual."""
    res = ctypes.c_void_p(1) if has_residual else None
    return int(lib().rmsnorm_bwd_workspace_size(T, heads, H, int(w_dtype), res, int(bool(deterministic))))


def rmsnorm_bwd_workspace_init(workspace, H: int, stream=None):
    _workspace(workspace, workspace.device)
    st_ = lib().rmsnorm_bwd_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                           H, _stream(workspace.device, stream))
    _check("rmsnorm_bwd_workspace_init", st_)


def rmsnorm_bwd_workspace(T: int, heads: int, H: int, device, deterministic=None, nbytes=None,
                          w_dtype: int = RMSN_W_BF16, has_residual=None):
    """A zero-filled (hence prepared) workspace tensor for rmsnorm_bwd.  With
    deterministic=None it serves both modes, with has_residual=None calls
    with and without dres (the largest of the sizes)."""
    torch = _torch()
    if nbytes is not None:
        n = nbytes
    else:
        modes = (True, False) if deterministic is None else (bool(deterministic),)
        resid = (False, True) if has_residual is None else (bool(has_residual),)
        sizes = [rmsnorm_bwd_workspace_size(T, heads, H, w_dtype, r, d) for d in modes for r in resid]
        n = 0 if min(sizes) == 0 else max(sizes)
    if n == 0:
        raise ValueError("unsupported shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def rmsnorm_bwd_route(T: int, heads: int, H: int, w_dtype: int, has_residual: bool,
                      deterministic: bool):
    """The route rmsnorm_bwd takes: (form, chunks, col_chunks, col_vecs, prefetch)."""
    r = RmsnRoute()
    _check("rmsnorm_bwd_route", lib().rmsnorm_bwd_route(T, heads, H, int(w_dtype), int(bool(has_residual)),
                                                        int(bool(deterministic)), ctypes.byref(r)))
    return int(r.form), int(r.chunks), int(r.col_chunks), int(r.col_vecs), int(r.prefetch)


def rmsnorm_gated_bwd_route(T: int, heads: int, H: int, w_dtype: int, deterministic: bool):
    """The route rmsnorm_gated_bwd takes: (form, chunks, col_chunks, col_vecs, prefetch)."""
    r = RmsnRoute()
    _check("rmsnorm_gated_bwd_route", lib().rmsnorm_gated_bwd_route(T, heads, H, int(w_dtype), int(bool(deterministic)),
                                                                    ctypes.byref(r)))
    return int(r.form), int(r.chunks), int(r.col_chunks), int(r.col_vecs), int(r.prefetch)


def rmsnorm_bwd_workspace_size_for_route(T: int, heads: int, H: int, route) -> int:
    return int(lib().rmsnorm_bwd_workspace_size_for_route(T, heads, H, RmsnRoute(*route)))


def _bwd_args(dy, x, rstd, w, residual, dx, dw):
    torch = _torch()
    _act(x, "x", x)
    T, heads, H, st, sh = geometry(x)
    for t, what in ((dy, "dy"), (residual, "residual")):
        _act(t, what, x)
        _same_geometry(x, t, what)
    dx = _like(x) if dx is None else dx
    _act(dx, "dx", x)
    _same_geometry(x, dx, "dx")
    _vec(rstd, "rstd", T * heads, (torch.float32,), x.device)
    _weight(w, H, x.device)
    if dw is None:
        dw = torch.empty(H, dtype=torch.float32, device=x.device)
    _vec(dw, "dw", H, (torch.float32,), x.device)
    return (T, heads, H, st, sh), dx, dw


def rmsnorm_bwd(dy, x, rstd, w, residual=None, deterministic: bool = True, *,
                dx=None, dw=None, workspace=None, stream=None):
    """dx (BF16) and dw (FP32) of the training RMSNorm backward.

    ``x`` is the forward's normalised input (h with a residual); ``residual``
    is the incoming gradient of h (dres) or None.  Returns (dx, dw)."""
    (T, heads, H, st, sh), dx, dw = _bwd_args(dy, x, rstd, w, residual, dx, dw)
    if workspace is None:
        workspace = rmsnorm_bwd_workspace(T, heads, H, x.device, deterministic, w_dtype=_w_dtype(w),
                                          has_residual=residual is not None)
    _workspace(workspace, x.device)
    st_ = lib().rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(rstd), _ptr(w), _w_dtype(w), _ptr(residual),
                            _ptr(dx), _ptr(dw), _ptr(workspace),
                            workspace.numel() * workspace.element_size(),
                            T, heads, H, st, sh, int(bool(deterministic)), _stream(x.device, stream))
    _check("rmsnorm_bwd", st_)
    return dx, dw


def rmsnorm_bwd_noalloc(dy, x, rstd, w, residual=None, deterministic: bool = True, *, dx, dw, stream=None):
    """rmsnorm_bwd on the library's own device scratch: no workspace, and no
    allocation by the library or here (dx and dw must be given)."""
    (T, heads, H, st, sh), dx, dw = _bwd_args(dy, x, rstd, w, residual, dx, dw)
    st_ = lib().rmsnorm_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(rstd), _ptr(w), _w_dtype(w), _ptr(residual),
                                    _ptr(dx), _ptr(dw), T, heads, H, st, sh, int(bool(deterministic)),
                                    _stream(x.device, stream))
    _check("rmsnorm_bwd_noalloc", st_)
    return dx, dw


def rmsnorm_bwd_routed(dy, x, rstd, w, route, residual=None, deterministic: bool = True, *,
                       dx=None, dw=None, workspace=None, stream=None):
    """rmsnorm_bwd with an explicit route: (form, chunks) or (form, chunks,
    0, 0, prefetch) for the pair and atomic forms, (form, chunks, col_chunks,
    col_vecs) for the column forms."""
    (T, heads, H, st, sh), dx, dw = _bwd_args(dy, x, rstd, w, residual, dx, dw)
    if workspace is None:
        workspace = rmsnorm_bwd_workspace(T, heads, H, x.device, deterministic,
                                          nbytes=rmsnorm_bwd_workspace_size_for_route(T, heads, H, route))
    _workspace(workspace, x.device)
    st_ = lib().rmsnorm_bwd_routed(_ptr(dy), _ptr(x), _ptr(rstd), _ptr(w), _w_dtype(w), _ptr(residual),
                                   _ptr(dx), _ptr(dw), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   T, heads, H, st, sh, int(bool(deterministic)), RmsnRoute(*route),
                                   _stream(x.device, stream))
    _check("rmsnorm_bwd_routed", st_)
    return dx, dw


# ---------------------------------------------------------- SiLU gate ----

def rmsnorm_gated_fwd(x, g, w, eps: float = 1e-6, deterministic: bool = True, *, y=None, rstd=None,
                      stream=None):
    """y = bf16(RMSNorm(x) * w * silu(g)) and rstd.  Returns (y, rstd)."""
    torch = _torch()
    _act(x, "x", x)
    T, heads, H, st, sh = geometry(x)
    _act(g, "g", x)
    _same_geometry(x, g, "g")
    y = _like(x) if y is None else y
    _act(y, "y", x)
    _same_geometry(x, y, "y")
    _weight(w, H, x.device)
    if rstd is None:
        rstd = torch.empty(T * heads, dtype=torch.float32, device=x.device)
    _vec(rstd, "rstd", T * heads, (torch.float32,), x.device)
    _check("rmsnorm_gated_fwd", lib().rmsnorm_gated_fwd(
        _ptr(x), _ptr(g), _ptr(w), _w_dtype(w), _ptr(y), _ptr(rstd), T, heads, H, st, sh, float(eps),
        int(bool(deterministic)), _stream(x.device, stream)))
    return y, rstd


def rmsnorm_gated_bwd(dy, x, g, rstd, w, deterministic: bool = True, *, dx=None, dg=None, dw=None,
                      workspace=None, stream=None):
    """dx, dg (BF16) and dw (FP32) of the gated forward.  Returns (dx, dg, dw)."""
    (T, heads, H, st, sh), dx, dw = _bwd_args(dy, x, rstd, w, None, dx, dw)
    _act(g, "g", x)
    _same_geometry(x, g, "g")
    dg = _like(x) if dg is None else dg
    _act(dg, "dg", x)
    _same_geometry(x, dg, "dg")
    if workspace is None:
        workspace = rmsnorm_bwd_workspace(T, heads, H, x.device, deterministic, w_dtype=_w_dtype(w))
    _workspace(workspace, x.device)
    _check("rmsnorm_gated_bwd", lib().rmsnorm_gated_bwd(
        _ptr(dy), _ptr(x), _ptr(g), _ptr(rstd), _ptr(w), _w_dtype(w), _ptr(dx), _ptr(dg), _ptr(dw),
        _ptr(workspace), workspace.numel() * workspace.element_size(), T, heads, H, st, sh,
        int(bool(deterministic)), _stream(x.device, stream)))
    return dx, dg, dw
