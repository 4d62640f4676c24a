"""NumPy front end of the FP64 CPU oracle for training RMSNorm (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; the library never imports it.
It shares no code with the HIP path.  Arrays of BF16 values travel as their
``uint16`` bit patterns.  Rows are contiguous ``[R, H]``; a strided per-head
view is gathered into rows by the caller before it gets here.

What each function computes, with the passages it follows, is written in the
header of oracle.c.  Parity pins: every function below is pinned by
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


# The mutation tests point this at deliberately broken copies of oracle.c to
# show that the pins catch them.
_LIB_OVERRIDE = os.environ.get("RMSNORM_ORACLE_LIB")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_OVERRIDE or _build.LIB
    if not _LIB_OVERRIDE and not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_round_array.argtypes = [_i64, _ptr, _ptr]
    lib.oracle_bf16_round_array.restype = None
    lib.oracle_fwd_f64.argtypes = [_i64, _i64, _ptr, _ptr, ctypes.c_double, _ptr, _ptr]
    lib.oracle_fwd_f64.restype = None
    lib.oracle_bwd_f64.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr]
    lib.oracle_bwd_f64.restype = None
    lib.oracle_residual_add.argtypes = [_i64, _ptr, _ptr, _ptr]
    lib.oracle_residual_add.restype = None
    lib.oracle_fwd_bf16.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, ctypes.c_int,
                                    ctypes.c_double, _ptr, _ptr, _ptr]
    lib.oracle_fwd_bf16.restype = ctypes.c_int
    lib.oracle_bwd_bf16.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, ctypes.c_int, _ptr,
                                    _ptr, _ptr, _ptr, _ptr]
    lib.oracle_bwd_bf16.restype = ctypes.c_int
    lib.oracle_dw_bf16.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, _ptr]
    lib.oracle_dw_bf16.restype = None
    lib.oracle_gated_fwd_f64.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, ctypes.c_double, _ptr, _ptr]
    lib.oracle_gated_fwd_f64.restype = None
    lib.oracle_gated_bwd_f64.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr]
    lib.oracle_gated_bwd_f64.restype = None
    lib.oracle_gated_fwd_bf16.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, ctypes.c_int, ctypes.c_double,
                                          _ptr, _ptr]
    lib.oracle_gated_fwd_bf16.restype = ctypes.c_int
    lib.oracle_gated_bwd_bf16.argtypes = [_i64, _i64, _ptr, _ptr, _ptr, _ptr, ctypes.c_int, _ptr,
                                          _ptr, _ptr, _ptr, _ptr, _ptr]
    lib.oracle_gated_bwd_bf16.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def num_threads() -> int:
    return _load().oracle_num_threads()


# ------------------------------------------------------------------ BF16 ----

def bf16_round(v) -> np.ndarray:
    """Round float64 values to BF16 (ties to even, one rounding); uint16 bits."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_bf16_round_array(v.size, _p(v), _p(out))
    return out


def bf16_to_f64(b) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ FP64 core ----

def fwd_f64(u: np.ndarray, w: np.ndarray, eps: float):
    """y and rstd of FP64 rows u[R,H] with weight w[H]."""
    u = _c(u, np.float64)
    w = _c(w, np.float64)
    R, H = u.shape
    y = np.empty_like(u)
    rstd = np.empty(R, dtype=np.float64)
    _load().oracle_fwd_f64(R, H, _p(u), _p(w), float(eps), _p(y), _p(rstd))
    return y, rstd


def bwd_f64(u, dy, w, rho, dres=None):
    """dx[R,H] and dw[H] of FP64 rows at the per-row rho (dres optional)."""
    u = _c(u, np.float64)
    dy = _c(dy, np.float64)
    w = _c(w, np.float64)
    rho = _c(rho, np.float64)
    dres = _c(dres, np.float64)
    R, H = u.shape
    dx = np.empty_like(u)
    dw = np.empty(H, dtype=np.float64)
    _load().oracle_bwd_f64(R, H, _p(u), _p(dy), _p(w), _p(rho), _p(dres), _p(dx), _p(dw))
    return dx, dw


# ----------------------------------------------------- BF16 storage path ----

def residual_add(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    r = _c(r, np.uint16)
    h = np.empty_like(x)
    _load().oracle_residual_add(x.size, _p(x), _p(r), _p(h))
    return h


def _weight(w):
    w = np.ascontiguousarray(w)
    if w.dtype == np.uint16:
        return w, 0
    if w.dtype == np.float32:
        return w, 1
    raise TypeError("w must be BF16 bits (uint16) or float32")


def fwd_bf16(x: np.ndarray, w: np.ndarray, eps: float, r: np.ndarray | None = None):
    """Forward from BF16 rows x[R,H] (uint16 bits), optional residual r.

    Returns (y bf16 bits, h bf16 bits or None, rstd float64)."""
    x = _c(x, np.uint16)
    r = _c(r, np.uint16)
    w, w32 = _weight(w)
    R, H = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x) if r is not None else None
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().oracle_fwd_bf16(R, H, _p(x), _p(r), _p(w), w32, float(eps), _p(y), _p(h), _p(rstd))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd_bf16 failed ({rc})")
    return y, h, rstd


def bwd_bf16(u: np.ndarray, dy: np.ndarray, w: np.ndarray, rho32: np.ndarray,
             dres: np.ndarray | None = None, want_dx64: bool = False):
    """Backward from BF16 rows at the kernel's FP32 rstd rho32[R].

    Returns (dx bf16 bits, dx64 float64 or None, dw float64)."""
    u = _c(u, np.uint16)
    dy = _c(dy, np.uint16)
    dres = _c(dres, np.uint16)
    rho32 = _c(rho32, np.float32)
    w, w32 = _weight(w)
    R, H = u.shape
    dx = np.empty_like(u)
    dx64 = np.empty(u.shape, dtype=np.float64) if want_dx64 else None
    dw = np.empty(H, dtype=np.float64)
    rc = _load().oracle_bwd_bf16(R, H, _p(u), _p(dy), _p(w), w32, _p(rho32), _p(dres),
                                 _p(dx), _p(dx64), _p(dw))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd_bf16 failed ({rc})")
    return dx, dx64, dw


def dw_bf16(u: np.ndarray, dy: np.ndarray, rho32: np.ndarray) -> np.ndarray:
    """dw alone (FP64) from BF16 rows at the kernel's FP32 rstd."""
    u = _c(u, np.uint16)
    dy = _c(dy, np.uint16)
    rho32 = _c(rho32, np.float32)
    R, H = u.shape
    dw = np.empty(H, dtype=np.float64)
    _load().oracle_dw_bf16(R, H, _p(u), _p(dy), _p(rho32), _p(dw))
    return dw


# --------------------------------------------------------- SiLU-gated ----

def gated_fwd_f64(u, g, w, eps):
    """Gated y and rstd of FP64 rows u[R,H] with gate g[R,H] and weight w[H]."""
    u, g, w = _c(u, np.float64), _c(g, np.float64), _c(w, np.float64)
    R, H = u.shape
    y = np.empty_like(u)
    rstd = np.empty(R, dtype=np.float64)
    _load().oracle_gated_fwd_f64(R, H, _p(u), _p(g), _p(w), float(eps), _p(y), _p(rstd))
    return y, rstd


def gated_bwd_f64(u, g, dy, w, rho):
    """Gated dx, dg and dw of FP64 rows at the per-row rho."""
    u, g, dy = _c(u, np.float64), _c(g, np.float64), _c(dy, np.float64)
    w, rho = _c(w, np.float64), _c(rho, np.float64)
    R, H = u.shape
    dx, dg = np.empty_like(u), np.empty_like(u)
    dw = np.empty(H, dtype=np.float64)
    _load().oracle_gated_bwd_f64(R, H, _p(u), _p(g), _p(dy), _p(w), _p(rho), _p(dx), _p(dg), _p(dw))
    return dx, dg, dw


def gated_fwd_bf16(x: np.ndarray, g: np.ndarray, w: np.ndarray, eps: float):
    """Gated forward from BF16 rows x, gate g: (y bf16 bits, rstd float64)."""
    x = _c(x, np.uint16)
    g = _c(g, np.uint16)
    w, w32 = _weight(w)
    R, H = x.shape
    y = np.empty_like(x)
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().oracle_gated_fwd_bf16(R, H, _p(x), _p(g), _p(w), w32, float(eps), _p(y), _p(rstd))
    if rc != 0:
        raise RuntimeError(f"oracle_gated_fwd_bf16 failed ({rc})")
    return y, rstd


def gated_bwd_bf16(u: np.ndarray, g: np.ndarray, dy: np.ndarray, w: np.ndarray, rho32: np.ndarray,
                   want_f64: bool = False):
    """Gated backward at the kernel's FP32 rstd.

    Returns (dx bits, dg bits, dx64 or None, dg64 or None, dw float64)."""
    u = _c(u, np.uint16)
    g = _c(g, np.uint16)
    dy = _c(dy, np.uint16)
    rho32 = _c(rho32, np.float32)
    w, w32 = _weight(w)
    R, H = u.shape
    dx, dg = np.empty_like(u), np.empty_like(u)
    dx64 = np.empty(u.shape, dtype=np.float64) if want_f64 else None
    dg64 = np.empty(u.shape, dtype=np.float64) if want_f64 else None
    dw = np.empty(H, dtype=np.float64)
    rc = _load().oracle_gated_bwd_bf16(R, H, _p(u), _p(g), _p(dy), _p(w), w32, _p(rho32), _p(dx), _p(dg),
                                       _p(dx64), _p(dg64), _p(dw))
    if rc != 0:
        raise RuntimeError(f"oracle_gated_bwd_bf16 failed ({rc})")
    return dx, dg, dx64, dg64, dw
