"""ctypes wrappers around liboracle.so (test infrastructure; see oracle/__init__.py).

All functions take and return numpy arrays on the host.  fp16 tensors are passed
as their raw 16-bit patterns; the C side decodes them itself.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from . import build as _build

_lib = None
_lock = threading.Lock()

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):
                _build.build()
            L = ctypes.CDLL(_build.LIB)
            L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
            L.oracle_half_to_double.restype = ctypes.c_double
            L.oracle_gemv.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p]
            L.oracle_gemv.restype = None
            L.oracle_gemv_t2.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p]
            L.oracle_gemv_t2.restype = None
            L.oracle_pm1.argtypes = [_p, _p, _i64, _i64, _i64, _p]
            L.oracle_pm1.restype = None
            L.oracle_xor_patch.argtypes = [_p, _i64, _i64, _p, _i64]
            L.oracle_xor_patch.restype = _i64
            L.oracle_xor_bits.argtypes = [_p, _p, _p, _i64, _p, _i64]
            L.oracle_xor_bits.restype = _i64
            L.oracle_rank_rows.argtypes = [_p, _i64, _i64, _p, _p]
            L.oracle_rank_rows.restype = None
            L.oracle_max_threads.restype = ctypes.c_int
            L.oracle_set_threads.argtypes = [ctypes.c_int]
            _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h) & 0xFFFF)


def gemv(x: np.ndarray, W: np.ndarray, S: np.ndarray, group: int = 128):
    """fp64 dequantise-and-dot.

    x: fp16 [M][K]; W: uint32 [N][ceil(K/32)]; S: fp16 [N][K/group].
    Returns (y, nrm), both float64 [M][N]: y = sum_k s*w*x, nrm = sum_k |s*x|.
    """
    x = np.ascontiguousarray(x, dtype=np.float16)
    W = np.ascontiguousarray(W, dtype=np.uint32)
    S = np.ascontiguousarray(S, dtype=np.float16)
    M, K = x.shape
    N = W.shape[0]
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if W.shape[1] != (K + 31) // 32 or S.shape != (N, K // group):
        raise ValueError("shape mismatch")
    y = np.empty((M, N), np.float64)
    nrm = np.empty((M, N), np.float64)
    lib().oracle_gemv(_ptr(x), _ptr(W), _ptr(S), M, K, N, group, _ptr(y), _ptr(nrm))
    return y, nrm


def gemv_rows(x, W, S, rows, group: int = 128):
    """The oracle at selected output rows only: returns (y, nrm) of shape [M][len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemv(x, W[rows], S[rows], group)


def gemv_t2(x: np.ndarray, T: np.ndarray, S: np.ndarray, group: int = 128):
    """fp64 ternary dequantise-and-dot.  x: fp16 [M][K]; T: uint32 [N][ceil(K/16)] of 2-bit
    slots; S: fp16 [N][K/group].  Returns (y, nrm) float64 [M][N], nrm = sum_k |s*t*x|."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    T = np.ascontiguousarray(T, dtype=np.uint32)
    S = np.ascontiguousarray(S, dtype=np.float16)
    M, K = x.shape
    N = T.shape[0]
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if T.shape[1] != (K + 15) // 16 or S.shape != (N, K // group):
        raise ValueError("shape mismatch")
    y = np.empty((M, N), np.float64)
    nrm = np.empty((M, N), np.float64)
    lib().oracle_gemv_t2(_ptr(x), _ptr(T), _ptr(S), M, K, N, group, _ptr(y), _ptr(nrm))
    return y, nrm


def gemv_t2_rows(x, T, S, rows, group: int = 128):
    rows = np.asarray(rows, dtype=np.int64)
    return gemv_t2(x, T[rows], S[rows], group)


def pm1(A: np.ndarray, W: np.ndarray, K: int) -> np.ndarray:
    """Exact +-1 product: A uint32 [M][K/32], W uint32 [N][K/32] -> int64 [M][N]."""
    A = np.ascontiguousarray(A, dtype=np.uint32)
    W = np.ascontiguousarray(W, dtype=np.uint32)
    M, N = A.shape[0], W.shape[0]
    y = np.empty((M, N), np.int64)
    lib().oracle_pm1(_ptr(A), _ptr(W), M, K, N, _ptr(y))
    return y


def xor_patch(W: np.ndarray, rows, K: int) -> tuple:
    """Returns (patched copy of W, number of out-of-range entries skipped)."""
    out = np.array(W, dtype=np.uint32, copy=True, order="C")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    bad = lib().oracle_xor_patch(_ptr(out), K, out.shape[0], _ptr(rows), rows.size)
    return out, int(bad)


def xor_bits(mats, entries) -> tuple:
    """Bit-granular patch: mats is a list of uint32 [N_i][K_i/32] arrays, entries int32 [n][3]
    of (matrix id, row, k).  Returns (patched copies, number of entries skipped)."""
    outs = [np.array(m, dtype=np.uint32, copy=True, order="C") for m in mats]
    ptrs = (ctypes.c_void_p * len(outs))(*[o.ctypes.data for o in outs])
    K = np.array([o.shape[1] * 32 for o in outs], np.int64)
    N = np.array([o.shape[0] for o in outs], np.int64)
    e = np.ascontiguousarray(np.asarray(entries, dtype=np.int32).reshape(-1, 3))
    bad = lib().oracle_xor_bits(ptrs, _ptr(K), _ptr(N), len(outs), _ptr(e), e.shape[0])
    return outs, int(bad)


def rank_rows(S: np.ndarray) -> tuple:
    """Exact scale ranking: S fp16 [N][G].  Returns (score int64 [N] in units of 2^-24,
    order int32 [N]: rows by score descending, ties by ascending row)."""
    S = np.ascontiguousarray(S, dtype=np.float16)
    N, G = S.shape
    score = np.empty(N, np.int64)
    order = np.empty(N, np.int32)
    lib().oracle_rank_rows(_ptr(S), N, G, _ptr(score), _ptr(order))
    return score, order


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))
