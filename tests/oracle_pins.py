"""Pins for the CPU oracle: facts about C = A·B that do not come from the oracle.

Each pin takes ``gemm(A, B) -> (C, T)`` (float32 row-major in, float64 out)
and raises AssertionError when the implementation under test disagrees with
what mathematics fixes.  ``test_oracle.py`` runs them on the real oracle and,
to show they have teeth, on copies of the oracle with a planted mistake.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import seedgen

U53 = 2.0 ** -53


def _eye(n: int, ld: int | None = None, fill: float = 0.0) -> np.ndarray:
    ld = n if ld is None else ld
    e = np.full((n, ld), fill, dtype=np.float32)
    e[:, :n] = 0.0
    e[np.arange(n), np.arange(n)] = 1.0
    return e


def pin_identity(gemm) -> None:
    """A = I gives C = B and B = I gives C = A, bit for bit, on non-square
    shapes with leading dimensions wider than the rows (wrong index, stride or
    operand order changes the result)."""
    for (m, n, k, seed) in [(7, 5, 7, 11), (13, 9, 13, 12), (33, 17, 33, 13)]:
        B = seedgen.matrix(k, n, "uniform", seed, ld=n + 3)
        C, T = gemm(_eye(k, ld=k + 2), B[:, :n], M=k, N=n, K=k)
        assert np.array_equal(C, B[:, :n].astype(np.float64)), "I*B != B"
        assert np.array_equal(T, np.abs(B[:, :n]).astype(np.float64))
    for (m, n, k, seed) in [(5, 7, 7, 21), (9, 13, 13, 22), (40, 33, 33, 23)]:
        A = seedgen.matrix(m, k, "normal", seed, ld=k + 5)
        C, T = gemm(A[:, :k], _eye(n, ld=n + 1), M=m, N=n, K=k)
        assert np.array_equal(C, A[:, :k].astype(np.float64)), "A*I != A"
        assert np.array_equal(T, np.abs(A[:, :k]).astype(np.float64))


def pin_all_ones(gemm) -> None:
    """All-ones M x K times all-ones K x N is K in every element, exactly."""
    for (m, n, k) in [(1, 1, 1), (3, 4, 5), (17, 31, 129), (64, 3, 1000)]:
        C, T = gemm(np.ones((m, k), np.float32), np.ones((k, n), np.float32))
        assert C.shape == (m, n)
        assert np.all(C == k), f"ones: expected {k}"
        assert np.all(T == k)


def pin_closed_forms(gemm) -> None:
    """Rank-1 and power-sum products with known closed forms (all exact)."""
    rng_x = seedgen.integer_matrix(1, 11, -7, 7, 31)[0]
    rng_y = seedgen.integer_matrix(1, 6, -9, 9, 32)[0]
    for k in (1, 2, 9, 100):
        A = np.repeat(rng_x[:, None], k, axis=1).astype(np.float32)
        B = np.repeat(rng_y[None, :], k, axis=0).astype(np.float32)
        C, T = gemm(A, B)
        assert np.array_equal(C, k * np.outer(rng_x, rng_y).astype(np.float64))
        assert np.array_equal(
            T, k * np.outer(np.abs(rng_x), np.abs(rng_y)).astype(np.float64))
    for k in (1, 2, 3, 10, 256, 777):
        kk = np.arange(1, k + 1, dtype=np.float32)
        A = np.tile(kk, (3, 1))                      # A[i][k] = k + 1
        C, _ = gemm(A, np.ones((k, 4), np.float32))  # sum of 1..K
        assert np.all(C == k * (k + 1) // 2)
        C, _ = gemm(A, np.tile(kk[:, None], (1, 5)))  # sum of squares
        assert np.all(C == k * (k + 1) * (2 * k + 1) // 6)
    for k in (1, 2, 5, 6, 99):
        # alternating signs: C = K mod 2, T = K (a sign or |.| slip shows)
        A = ((-1.0) ** np.arange(k)).astype(np.float32)[None, :]
        C, T = gemm(A, np.ones((k, 2), np.float32))
        assert np.all(C == (k % 2)) and np.all(T == k)


def _exact(A: np.ndarray, B: np.ndarray):
    m, k = A.shape
    n = B.shape[1]
    C = [[sum((Fraction(float(A[i, t])) * Fraction(float(B[t, j]))
               for t in range(k)), Fraction(0)) for j in range(n)]
         for i in range(m)]
    T = [[sum((abs(Fraction(float(A[i, t]))) * abs(Fraction(float(B[t, j])))
               for t in range(k)), Fraction(0)) for j in range(n)]
         for i in range(m)]
    return C, T


def pin_brute_force(gemm) -> None:
    """Every shape with M, N, K in 1..4 (and a few to 6) on random floats,
    against exact rational sums: |C - exact| <= K * 2**-53 * T."""
    shapes = [(m, n, k) for m in range(1, 5) for n in range(1, 5)
              for k in range(1, 5)] + [(6, 5, 6), (5, 6, 3), (2, 3, 6)]
    for idx, (m, n, k) in enumerate(shapes):
        A, B = seedgen.gemm_inputs(m, n, k, "normal" if idx % 2 else "uniform",
                                   1000 + idx)
        C, T = gemm(A, B)
        assert np.all(np.isfinite(C)) and np.all(np.isfinite(T))
        Ce, Te = _exact(A, B)
        for i in range(m):
            for j in range(n):
                bound = Fraction(k) * Fraction(U53) * Te[i][j]
                assert abs(Fraction(float(C[i, j])) - Ce[i][j]) <= bound, \
                    (m, n, k, i, j)
                assert abs(Fraction(float(T[i, j])) - Te[i][j]) <= bound


def pin_numpy(gemm) -> None:
    """Agreement with numpy's float64 product on upcast inputs within the
    float64 accumulation bound of two different summation orders."""
    for (m, n, k, dist, seed) in [(37, 29, 61, "uniform", 41),
                                  (64, 128, 256, "normal", 42),
                                  (100, 150, 77, "uniform", 43)]:
        A, B = seedgen.gemm_inputs(m, n, k, dist, seed)
        C, T = gemm(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        tref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        assert np.all(np.abs(C - ref) <= 4 * k * U53 * tref)
        assert np.all(np.abs(T - tref) <= 4 * k * U53 * tref)


def pin_leading_dims(gemm) -> None:
    """NaN in the padding columns of A and B must never reach C."""
    m, n, k = 19, 23, 29
    A, B = seedgen.gemm_inputs(m, n, k, "uniform", 51, lda=k + 7,
                               ldb=n + 9, fill=np.nan)
    C, T = gemm(A[:, :k], B[:, :n], M=m, N=n, K=k)
    assert np.all(np.isfinite(C)) and np.all(np.isfinite(T))
    Cc, Tc = gemm(np.ascontiguousarray(A[:, :k]), np.ascontiguousarray(B[:, :n]))
    assert np.array_equal(C, Cc) and np.array_equal(T, Tc)


def pin_transpose(gemm) -> None:
    """(A·B)^T = B^T·A^T: the same products summed in the same k order."""
    A, B = seedgen.gemm_inputs(21, 34, 55, "normal", 61)
    C, T = gemm(A, B)
    Ct, Tt = gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T, Ct) and np.array_equal(T.T, Tt)


def pin_empty(gemm) -> None:
    """K = 0 is the empty sum; M = 0 or N = 0 gives an empty result."""
    C, T = gemm(np.zeros((3, 1), np.float32), np.zeros((1, 4), np.float32),
                M=3, N=4, K=0)
    assert C.shape == (3, 4) and np.all(C == 0) and np.all(T == 0)
    C, _ = gemm(np.zeros((0, 5), np.float32), np.ones((5, 6), np.float32))
    assert C.shape == (0, 6)
    C, _ = gemm(np.ones((4, 5), np.float32), np.zeros((5, 0), np.float32))
    assert C.shape == (4, 0)


ALL_PINS = [pin_identity, pin_all_ones, pin_closed_forms, pin_brute_force,
            pin_numpy, pin_leading_dims, pin_transpose, pin_empty]


# -- the transpose reference ------------------------------------------------
# Each takes ``tr(A, **kw) -> out`` with the signature of oracle.transpose.

def pin_transpose_numpy(tr) -> None:
    """Agreement, bit for bit, with numpy's transposed view on many shapes."""
    for (r, c, seed) in [(1, 1, 1), (1, 7, 2), (7, 1, 3), (13, 29, 4),
                         (64, 64, 5), (65, 63, 6), (200, 3, 7)]:
        A = seedgen.matrix(r, c, "normal", seed)
        assert np.array_equal(tr(A), np.ascontiguousarray(A.T))


def pin_transpose_index_form(tr) -> None:
    """in[i][j] = i * cols + j (exact integers) lands at out[j][i]."""
    r, c = 37, 53
    A = (np.arange(r)[:, None] * c + np.arange(c)[None, :]).astype(np.float32)
    out = tr(A)
    for j in range(c):
        for i in range(r):
            assert out[j, i] == i * c + j


def pin_transpose_leading_dims(tr) -> None:
    """Input gaps (NaN) are not read; output gaps keep their fill."""
    r, c = 9, 14
    A = seedgen.matrix(r, c, "uniform", 8, ld=c + 5, fill=np.nan)
    out = tr(A[:, :c], rows=r, cols=c, ldo=r + 3, fill=-5.0)
    assert out.shape == (c, r + 3)
    assert np.array_equal(out[:, :r], np.ascontiguousarray(A[:, :c].T))
    assert np.all(out[:, r:] == -5.0)


TRANSPOSE_PINS = [pin_transpose_numpy, pin_transpose_index_form,
                  pin_transpose_leading_dims]
