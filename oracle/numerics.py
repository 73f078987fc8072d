"""ctypes front of the oracle's C arithmetic (oracle/step.c). Test infrastructure."""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load(_build.LIB)
    return _lib


def load(path: str):
    """Load a build of oracle/step.c and declare its functions."""
    L = ctypes.CDLL(path)
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    vp = ctypes.c_void_p
    L.oracle_bias_correction.argtypes = [f32, i64]
    L.oracle_bias_correction.restype = f32
    L.oracle_threads.argtypes = []
    L.oracle_threads.restype = ctypes.c_int
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_set_threads.restype = None
    L.oracle_narrow.argtypes = [vp, i64, vp]
    L.oracle_widen.argtypes = [vp, i64, vp]
    L.oracle_reduce.argtypes = [i32, vp, f32, i64, vp]
    L.oracle_adam.argtypes = [i64, vp, vp, vp, vp, vp, vp]
    L.oracle_step.argtypes = [i32, vp, f32, i64, vp, vp, vp, vp, vp, vp, f32]
    L.oracle_norm_sq.argtypes = [i32, vp, f32, i64]
    L.oracle_norm_sq.restype = ctypes.c_double
    L.oracle_clip_coefficient.argtypes = [vp, i32, f32, vp]
    L.oracle_clip_coefficient.restype = f32
    for f in (L.oracle_narrow, L.oracle_widen, L.oracle_reduce, L.oracle_adam, L.oracle_step):
        f.restype = None
    return L


def _ptr(a):
    if a is None:
        return None
    if not a.flags.c_contiguous:
        raise ValueError("oracle arrays must be contiguous")
    return a.ctypes.data


def _check(a, dtype, n=None):
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    if n is not None and a.size != n:
        raise ValueError(f"expected {n} elements, got {a.size}")


def threads() -> int:
    return lib().oracle_threads()


def set_threads(n: int) -> None:
    """Threads of the element loops from now on (results do not depend on it)."""
    lib().oracle_set_threads(int(n))


def bias_correction(beta: float, t: int) -> float:
    return float(lib().oracle_bias_correction(beta, t))


def narrow(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_narrow(_ptr(x), x.size, _ptr(out))
    return out


def widen(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_widen(_ptr(h), h.size, _ptr(out))
    return out


def _rep_array(reps, n):
    arr = (ctypes.c_void_p * len(reps))()
    for j, r in enumerate(reps):
        _check(r, np.uint16, n)
        arr[j] = _ptr(r)
    return arr


def hp_array(hp: dict, step: int) -> np.ndarray:
    """{lr, b1, b2, eps, wd, bc1, bc2} as the C side takes them, for step t."""
    bc1 = bias_correction(hp["beta1"], step)
    bc2 = bias_correction(hp["beta2"], step)
    return np.array([hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], bc1, bc2],
                    dtype=np.float32)


def reduce(reps, scale: float, out: np.ndarray | None = None) -> np.ndarray:
    n = reps[0].size
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    _check(out, np.uint16, n)
    keep = list(reps)
    lib().oracle_reduce(len(keep), _rep_array(keep, n), scale, n, _ptr(out))
    return out


def adam(grad, master, m, v, hp_arr, param_out=None) -> None:
    n = grad.size
    _check(grad, np.uint16)
    for a in (master, m, v):
        _check(a, np.float32, n)
    if param_out is not None:
        _check(param_out, np.uint16, n)
    lib().oracle_adam(n, _ptr(grad), _ptr(master), _ptr(m), _ptr(v), _ptr(param_out), _ptr(hp_arr))


def norm_sq(reps, scale: float) -> float:
    """Sum of squares (fp64, element order) of the reduced gradient."""
    n = reps[0].size
    keep = list(reps)
    return float(lib().oracle_norm_sq(len(keep), _rep_array(keep, n), scale, n))


def clip_coefficient(parts, max_norm: float) -> tuple:
    """(coefficient as fp32, global norm) from the ranks' squared norms."""
    arr = np.ascontiguousarray(np.asarray(parts, dtype=np.float64))
    norm = ctypes.c_double()
    c = lib().oracle_clip_coefficient(_ptr(arr), arr.size, max_norm, ctypes.byref(norm))
    return float(np.float32(c)), norm.value


def step(reps, scale: float, master, m, v, hp_arr, param_out=None, main_grad_out=None,
         grad_coeff: float = 1.0) -> None:
    n = master.size
    for a in (master, m, v):
        _check(a, np.float32, n)
    if param_out is not None:
        _check(param_out, np.uint16, n)
    if main_grad_out is not None:
        _check(main_grad_out, np.float32, n)
    keep = list(reps)
    lib().oracle_step(len(keep), _rep_array(keep, n), scale, n, _ptr(master), _ptr(m), _ptr(v),
                      _ptr(param_out), _ptr(main_grad_out), _ptr(hp_arr), grad_coeff)
