"""CPU oracle for single-precision dense C = A * B (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and this package never imports the GPU library: the two share no
code.

What it computes follows amittech.dev, "3.5 Project: tiled matrix
multiplication", section "starter scaffolding" (the CPU reference routine):
each output is a row-of-A by column-of-B dot product, every product taken in
double from the float inputs and summed in double in ascending k.  The sum is
returned in double; ``(float)`` of it is the page's float-rounded reference.
The companion matrix S = sum_k |a_ik * b_kj| scales the error bound that the
checker in ``oracle.check`` applies.

The arithmetic lives in ``oracle.c`` (plain C, pthreads over whole output
rows, compiled with ``-ffp-contract=off``); this module only marshals numpy
arrays to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O3", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (always, unless force=False
    and the library is newer than its source)."""
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC)):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, vp, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_sgemm_f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, cint]
    lib.oracle_sgemm_f64.restype = cint
    lib.oracle_sgemm_rows_f64.argtypes = [i64, vp, i64, i64, vp, i64, vp, i64, vp, vp, i64, cint]
    lib.oracle_sgemm_rows_f64.restype = cint
    lib.oracle_sgemm_entries_f64.argtypes = [i64, vp, vp, i64, vp, i64, vp, i64, vp, vp]
    lib.oracle_sgemm_entries_f64.restype = cint
    lib.oracle_sgemm_ex_f64.argtypes = [cint, cint, i64, i64, i64, ctypes.c_double, vp, i64, vp, i64,
                                        ctypes.c_double, vp, i64, vp, vp, vp, i64]
    lib.oracle_sgemm_ex_f64.restype = cint
    lib.oracle_fma_chain_f32.argtypes = [i64, ctypes.c_float, ctypes.c_float, cint, vp]
    lib.oracle_fma_chain_f32.restype = None
    lib.oracle_mfma_probe_f64.argtypes = [i64, vp, vp, vp]
    lib.oracle_mfma_probe_f64.restype = None
    return lib


def default_threads() -> int:
    """Threads the oracle uses by default: every core this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ld(x: np.ndarray, name: str) -> int:
    """Leading dimension (in elements) of a 2-D row-major float32 view."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} must have unit column stride")
    if x.strides[0] % 4:
        raise ValueError(f"{name} row stride must be a whole number of floats")
    return max(x.strides[0] // 4, x.shape[1], 1)


def _ptr(x: np.ndarray) -> int:
    return x.__array_interface__["data"][0]


def sgemm_f64(A: np.ndarray, B: np.ndarray, bound: bool = True, threads: int | None = None,
              lib: ctypes.CDLL | None = None):
    """Full product in double: returns (C, S) with S None unless ``bound``.

    A is M x K and B is K x N (row-major float32 views; a row stride larger
    than the row length is the leading dimension)."""
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if bound else None
    rc = lib.oracle_sgemm_f64(M, N, K, _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"),
                              _ptr(C), _ptr(S) if bound else None, max(N, 1),
                              threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_sgemm_f64 failed")
    return C, S


def sgemm_rows_f64(A: np.ndarray, B: np.ndarray, rows, bound: bool = True,
                   threads: int | None = None, lib: ctypes.CDLL | None = None):
    """Whole rows ``rows`` of A*B in double: returns (C_rows, S_rows)."""
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise IndexError("row index out of range")
    C = np.empty((rows.size, N), dtype=np.float64)
    S = np.empty((rows.size, N), dtype=np.float64) if bound else None
    rc = lib.oracle_sgemm_rows_f64(rows.size, _ptr(rows), N, K, _ptr(A), _ld(A, "A"),
                                   _ptr(B), _ld(B, "B"), _ptr(C), _ptr(S) if bound else None,
                                   max(N, 1), threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_sgemm_rows_f64 failed")
    return C, S


def sgemm_entries_f64(A: np.ndarray, B: np.ndarray, rows, cols, lib: ctypes.CDLL | None = None):
    """Single elements (rows[t], cols[t]) of A*B in double: returns (vals, S)."""
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("index out of range")
    out = np.empty(rows.size, dtype=np.float64)
    S = np.empty(rows.size, dtype=np.float64)
    rc = lib.oracle_sgemm_entries_f64(rows.size, _ptr(rows), _ptr(cols), K, _ptr(A), _ld(A, "A"),
                                      _ptr(B), _ld(B, "B"), _ptr(out), _ptr(S))
    if rc != 0:
        raise RuntimeError("oracle_sgemm_entries_f64 failed")
    return out, S


def fma_chain_f32(iters: int, x: float, y: float, chains: int = 16, lib: ctypes.CDLL | None = None):
    """Final values of the compute probe's multiply-add chains (float32)."""
    lib = lib or load()
    out = np.empty(chains, dtype=np.float32)
    lib.oracle_fma_chain_f32(iters, x, y, chains, _ptr(out))
    return out


def mfma_probe_f64(iters: int, a_vals: np.ndarray, b_vals: np.ndarray, lib: ctypes.CDLL | None = None):
    """The 32 x 32 matrix the matrix-unit probe accumulates, in double."""
    lib = lib or load()
    a = np.ascontiguousarray(a_vals, dtype=np.float32)
    b = np.ascontiguousarray(b_vals, dtype=np.float32)
    if a.size != 64 or b.size != 64:
        raise ValueError("a_vals and b_vals hold 64 values each")
    D = np.empty((32, 32), dtype=np.float64)
    lib.oracle_mfma_probe_f64(iters, _ptr(a), _ptr(b), _ptr(D))
    return D


def sgemm_ex_f64(transa: bool, transb: bool, alpha: float, A: np.ndarray, B: np.ndarray,
                 beta: float, C0: np.ndarray | None, lib: ctypes.CDLL | None = None):
    """C = alpha op(A) op(B) + beta C0 in double (row-major).  A is stored
    M x K (or K x M when transa), B K x N (or N x K when transb).  Returns
    (C, S, E) with S = |alpha| sum|ab| and E = |alpha sum ab| + |beta C0|."""
    lib = lib or load()
    M, K = (A.shape[1], A.shape[0]) if transa else A.shape
    Kb, N = (B.shape[1], B.shape[0]) if transb else B.shape
    if Kb != K:
        raise ValueError("inner dimensions differ")
    if C0 is None:
        if beta != 0:
            raise ValueError("beta != 0 needs C0")
        C0 = np.zeros((max(M, 1), max(N, 1)), dtype=np.float32)
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    E = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_sgemm_ex_f64(int(transa), int(transb), M, N, K, float(alpha), _ptr(A), _ld(A, "A"),
                                 _ptr(B), _ld(B, "B"), float(beta), _ptr(C0), _ld(C0, "C0"),
                                 _ptr(C), _ptr(S), _ptr(E), max(N, 1))
    if rc != 0:
        raise RuntimeError("oracle_sgemm_ex_f64 failed")
    return C, S, E
