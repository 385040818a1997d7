"""Seeded synthetic matrices for the FP32 GEMM C = A·B.

This module only draws random numbers: it does no matrix arithmetic and is
shared, unchanged, by the CPU oracle's tests, the GPU parity tests, the smoke
run and the benchmark, so that every side sees the same bytes.

Generator: SplitMix64 in its counter form (Steele, Lea & Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014).  Draw number ``n``
of stream ``seed`` is ``mix64(seed + (n + 1) * 0x9E3779B97F4A7C15)`` where
``mix64`` is the published finaliser (xor-shift 30, multiply
0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31).

Distributions (the workloads name "uniform[-1,1)" and "normal(0,1)"):

* ``uniform``: ``m = x >> 40`` is a 24-bit integer and the value is
  ``m * 2**-23 - 1``.  That is exactly ``2u - 1`` for ``u = m * 2**-24`` in
  [0, 1), and it is exact in float32: -1 can occur, +1 cannot.
* ``normal``: Box-Muller in float64 from two 53-bit uniforms
  ``u1 = ((x0 >> 11) + 1) * 2**-53`` in (0, 1] and ``u2 = (x1 >> 11) * 2**-53``
  in [0, 1), ``z = sqrt(-2 ln u1) * cos(2 pi u2)``, rounded to float32.  Value
  ``n`` consumes draws ``2n`` and ``2n + 1``.

Matrix ``A`` (M x K) takes draws ``n = i*K + k``; matrix ``B`` (K x N) takes
draws ``n = M*K + k*N + j`` of the same seed (``gemm_inputs``).  Leading
dimensions larger than the logical width leave the padding columns to the
caller (``fill``).
"""
from __future__ import annotations

import hashlib

import numpy as np

__all__ = ["splitmix64", "draw", "matrix", "gemm_inputs", "sha256_of"]

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of stream ``seed`` as uint64."""
    x = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    x *= _GAMMA
    x += np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    y = x >> np.uint64(30)
    x ^= y
    x *= _M1
    np.right_shift(x, np.uint64(27), out=y)
    x ^= y
    x *= _M2
    np.right_shift(x, np.uint64(31), out=y)
    x ^= y
    return x


def _uniform_chunk(seed: int, start: int, count: int) -> np.ndarray:
    m = splitmix64(seed, start, count) >> np.uint64(40)
    v = m.astype(np.float32)
    v *= np.float32(2.0 ** -23)
    v -= np.float32(1.0)
    return v


def _normal_chunk(seed: int, start: int, count: int) -> np.ndarray:
    x = splitmix64(seed, 2 * start, 2 * count)
    x0 = x[0::2] >> np.uint64(11)
    x1 = x[1::2] >> np.uint64(11)
    u1 = (x0.astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = x1.astype(np.float64) * (2.0 ** -53)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return z.astype(np.float32)


def draw(dist: str, seed: int, start: int, count: int) -> np.ndarray:
    """``count`` float32 values of distribution ``dist`` from draw ``start``."""
    if dist == "uniform":
        fn = _uniform_chunk
    elif dist == "normal":
        fn = _normal_chunk
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    out = np.empty(count, dtype=np.float32)
    for s in range(0, count, _CHUNK):
        c = min(_CHUNK, count - s)
        out[s:s + c] = fn(seed, start + s, c)
    return out


def matrix(rows: int, cols: int, dist: str, seed: int, start: int = 0,
           ld: int | None = None, fill: float = np.nan) -> np.ndarray:
    """A ``rows x ld`` float32 array whose first ``cols`` columns hold draws
    ``start + r*cols + c``; columns ``cols .. ld-1`` are set to ``fill``."""
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld < cols")
    vals = draw(dist, seed, start, rows * cols).reshape(rows, cols)
    if ld == cols:
        return vals
    out = np.full((rows, ld), fill, dtype=np.float32)
    out[:, :cols] = vals
    return out


def gemm_inputs(M: int, N: int, K: int, dist: str, seed: int,
                lda: int | None = None, ldb: int | None = None,
                fill: float = np.nan) -> tuple[np.ndarray, np.ndarray]:
    """Seeded ``A`` (M x lda, logical M x K) and ``B`` (K x ldb, logical K x N)."""
    A = matrix(M, K, dist, seed, 0, lda, fill)
    B = matrix(K, N, dist, seed, M * K, ldb, fill)
    return A, B


def integer_matrix(rows: int, cols: int, lo: int, hi: int, seed: int,
                   start: int = 0) -> np.ndarray:
    """Integers uniform on [lo, hi] as float32 (for order-independent sums)."""
    span = hi - lo + 1
    x = splitmix64(seed, start, rows * cols)
    v = (x % np.uint64(span)).astype(np.int64) + lo
    return v.astype(np.float32).reshape(rows, cols)


def sha256_of(*arrays: np.ndarray) -> str:
    """Digest of the arrays' bytes, in order (recorded with results)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
