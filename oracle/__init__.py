"""CPU oracle for the fixed-order bf16 AllReduce -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path never routes through it, and it imports
nothing from the product package.

Two independent parts:
  * the C oracle (ar_oracle.c) -- the reduction as the pages define it,
    written out as a plain loop; loaded here through ctypes;
  * exact.py -- IEEE-754 rounding and addition from their definitions in
    exact rational arithmetic, used only to pin the C oracle.

Parity of every function here is pinned by tests/test_oracle.py.
"""
import ctypes
import os
import threading

import numpy as np

from . import build as _build

_lock = threading.Lock()
_lib = None


def lib():
    """Load (building on first use if absent) the C oracle library."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):
                _build.build()
            L = ctypes.CDLL(_build.LIB)
            L.oracle_f32_to_bf16.argtypes = [ctypes.c_uint32]
            L.oracle_f32_to_bf16.restype = ctypes.c_uint16
            L.oracle_f32_to_bf16_array.argtypes = [
                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            L.oracle_f32_to_bf16_array.restype = None
            L.oracle_f32_add_bits.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
            L.oracle_f32_add_bits.restype = ctypes.c_uint32
            L.oracle_allreduce_bf16.argtypes = [
                ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                ctypes.c_void_p, ctypes.c_int]
            L.oracle_allreduce_bf16.restype = None
            L.oracle_allreduce_f32.argtypes = [
                ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t,
                ctypes.c_void_p]
            L.oracle_allreduce_f32.restype = None
            L.oracle_max_threads.argtypes = []
            L.oracle_max_threads.restype = ctypes.c_int
            L.oracle_gemv_f64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int]
            L.oracle_gemv_f64.restype = None
            L.oracle_add_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_void_p]
            L.oracle_add_rmsnorm.restype = None
            L.oracle_sum_abs_f64.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                             ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
            L.oracle_sum_abs_f64.restype = None
            _lib = L
        return _lib


def _rank_ptrs(ranks):
    arrs = [np.ascontiguousarray(r, dtype=np.uint16) for r in ranks]
    n = arrs[0].size
    for a in arrs:
        if a.size != n:
            raise ValueError("rank buffers differ in length")
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    return arrs, ptrs, n


def allreduce(ranks, threads: int = 1) -> np.ndarray:
    """Fixed rank-order fp32 sum of bf16 rank buffers, rounded to bf16.

    ranks: sequence of N uint16 arrays (bf16 bit patterns), equal length n.
    Returns uint16 [N, n]: every rank's copy of the reduced vector.
    """
    arrs, ptrs, n = _rank_ptrs(ranks)
    out = np.empty((len(arrs), n), dtype=np.uint16)
    if n:
        lib().oracle_allreduce_bf16(ptrs, len(arrs), n, out.ctypes.data, int(threads))
    return out


def allreduce_f32(ranks) -> np.ndarray:
    """The binary32 accumulator of the same fold, before rounding: float32 [n]."""
    arrs, ptrs, n = _rank_ptrs(ranks)
    acc = np.empty(n, dtype=np.float32)
    if n:
        lib().oracle_allreduce_f32(ptrs, len(arrs), n, acc.ctypes.data)
    return acc


def f32_to_bf16(bits32: int) -> int:
    return int(lib().oracle_f32_to_bf16(int(bits32) & 0xFFFFFFFF))


def f32_to_bf16_array(bits32) -> np.ndarray:
    a = np.ascontiguousarray(bits32, dtype=np.uint32)
    out = np.empty(a.size, dtype=np.uint16)
    if a.size:
        lib().oracle_f32_to_bf16_array(a.ctypes.data, a.size, out.ctypes.data)
    return out


def f32_add_bits(a: int, b: int) -> int:
    return int(lib().oracle_f32_add_bits(int(a) & 0xFFFFFFFF, int(b) & 0xFFFFFFFF))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def gemv(W, x, threads=0):
    """y[m] = sum_k W[m,k] * x[k] for bf16 patterns W [M, K] and x [K], as
    binary64 (the exact products summed in order; see ar_oracle.c)."""
    W = np.ascontiguousarray(W, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = W.shape
    assert x.shape == (K,)
    y = np.empty(M, dtype=np.float64)
    lib().oracle_gemv_f64(W.ctypes.data, x.ctypes.data, M, K, y.ctypes.data, int(threads))
    return y


def add_rmsnorm(a, res, gamma, eps):
    """Residual add and RMS norm after the AllReduce (see ar_oracle.c):
    returns (h bf16 patterns, y as unrounded binary64)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    res = np.ascontiguousarray(res, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    n = a.size
    assert res.size == n and gamma.size == n
    h = np.empty(n, dtype=np.uint16)
    y = np.empty(n, dtype=np.float64)
    lib().oracle_add_rmsnorm(a.ctypes.data, res.ctypes.data, gamma.ctypes.data, n, float(eps),
                             h.ctypes.data, y.ctypes.data)
    return h, y


def sum_abs(inputs):
    """Per element, the binary64 sum over ranks and the sum of magnitudes
    (reference of the arrival-order atomic variant; see ar_oracle.c):
    returns (sum, abs_sum), float64 [n] each."""
    arrs = [np.ascontiguousarray(x, dtype=np.uint16) for x in inputs]
    N = len(arrs)
    n = arrs[0].size
    ptrs = (ctypes.c_void_p * N)(*[a.ctypes.data for a in arrs])
    s = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    lib().oracle_sum_abs_f64(ptrs, N, n, s.ctypes.data, a.ctypes.data)
    return s, a
