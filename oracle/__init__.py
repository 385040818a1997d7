"""CPU oracle for C = A·B in float64 (see ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library or its binding.

``gemm(A, B, M=None, N=None, K=None)`` takes float32 numpy arrays in row-major
storage (``A`` is M x lda, ``B`` is K x ldb, leading dimension = row length of
the array, logical extents given or taken from the shapes) and returns
``(C, T)``: float64 arrays of shape (M, N) holding the exact-order double sums
``C[i,j] = sum_k A[i,k] B[k,j]`` and ``T[i,j] = sum_k |A[i,k]| |B[k,j]|``.

Parity is pinned, not assumed: ``tests/test_oracle.py`` checks it against
identity products, all-ones and rank-1 closed forms, exact rational brute
force on tiny shapes, numpy's float64 product and leading-dimension sentinels.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import build as _build

__all__ = ["gemm", "transpose", "max_threads", "library_path", "load_library"]

_lib = None


def load_library(path: str):
    """ctypes handle on an oracle build at ``path`` (with prototypes set)."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    fp = ctypes.c_void_p
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, fp, i64, fp, i64,
                                    fp, i64, fp, i64, ctypes.c_int]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_transpose_f32.argtypes = [i64, i64, fp, i64, fp, i64]
    lib.oracle_transpose_f32.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = load_library(_build.ensure_built())
    return _lib


def library_path() -> str:
    return _build.LIB


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _rowmajor(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return x
    if (x.shape[1] > 1 and x.strides[1] != 4) or x.strides[0] % 4 != 0:
        raise ValueError(f"{name} must be row-major with unit column stride")
    return x


def gemm(A: np.ndarray, B: np.ndarray, M: int | None = None,
         N: int | None = None, K: int | None = None,
         with_t: bool = True, threads: int = 0, lib=None):
    """float64 ``(C, T)`` of the logical M x K by K x N product (T is None
    when ``with_t`` is false).  ``lib`` selects another build (tests only)."""
    A = _rowmajor(A, "A")
    B = _rowmajor(B, "B")
    M = A.shape[0] if M is None else M
    K = B.shape[0] if K is None else K
    N = B.shape[1] if N is None else N
    lda = A.strides[0] // 4 if A.shape[0] > 1 else max(A.shape[1], 1)
    ldb = B.strides[0] // 4 if B.shape[0] > 1 else max(B.shape[1], 1)
    if A.shape[0] < M or A.shape[1] < K or B.shape[0] < K or B.shape[1] < N:
        raise ValueError("logical extents exceed the arrays")
    # Outputs start as NaN so that an element the C code fails to write shows.
    C = np.full((M, N), np.nan, dtype=np.float64)
    T = np.full((M, N), np.nan, dtype=np.float64) if with_t else None
    ldc = max(N, 1)
    lib = _load() if lib is None else lib
    rc = lib.oracle_gemm_f64(
        M, N, K, A.ctypes.data, max(lda, K, 1), B.ctypes.data, max(ldb, N, 1),
        C.ctypes.data, ldc, T.ctypes.data if with_t else None, ldc,
        int(threads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_f64 rejected the arguments (rc={rc})")
    return C, T


def transpose(A: np.ndarray, rows: int | None = None, cols: int | None = None,
              ldo: int | None = None, fill: float = np.nan, lib=None) -> np.ndarray:
    """The ``cols x ldo`` float32 array whose first ``rows`` columns hold
    ``A[:rows, :cols]`` transposed; the gap columns keep ``fill``."""
    A = _rowmajor(A, "A")
    rows = A.shape[0] if rows is None else rows
    cols = A.shape[1] if cols is None else cols
    ldo = max(rows, 1) if ldo is None else ldo
    ldi = A.strides[0] // 4 if A.shape[0] > 1 else max(A.shape[1], 1)
    out = np.full((cols, ldo), fill, dtype=np.float32)
    lib = _load() if lib is None else lib
    rc = lib.oracle_transpose_f32(rows, cols, A.ctypes.data, max(ldi, cols, 1),
                                  out.ctypes.data, ldo)
    if rc != 0:
        raise ValueError(f"oracle_transpose_f32 rejected the arguments (rc={rc})")
    return out
