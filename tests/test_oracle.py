"""The CPU oracle against facts that do not come from it (CPU only)."""
from __future__ import annotations

import os
import re

import numpy as np
import pytest

import oracle
import seedgen
from oracle import build as oracle_build

from oracle_pins import ALL_PINS, TRANSPOSE_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle_mod, pin):
    pin(oracle_mod.gemm)


def test_thread_count_does_not_change_bits(oracle_mod):
    A, B = seedgen.gemm_inputs(67, 45, 301, "normal", 71)
    C1, T1 = oracle_mod.gemm(A, B, threads=1)
    C8, T8 = oracle_mod.gemm(A, B, threads=max(2, oracle_mod.max_threads()))
    assert np.array_equal(C1, C8) and np.array_equal(T1, T8)


def test_rejects_bad_arguments(oracle_mod):
    lib = oracle_mod.load_library(oracle_mod.library_path())
    buf = np.zeros(64, np.float32)
    out = np.zeros(64, np.float64)
    p, o = buf.ctypes.data, out.ctypes.data
    assert lib.oracle_gemm_f64(-1, 2, 2, p, 2, p, 2, o, 2, o, 2, 1) == -1
    assert lib.oracle_gemm_f64(2, 2, 3, p, 2, p, 2, o, 2, o, 2, 1) == -1  # lda<K
    assert lib.oracle_gemm_f64(2, 3, 2, p, 2, p, 2, o, 3, o, 3, 1) == -1  # ldb<N
    assert lib.oracle_gemm_f64(2, 3, 2, p, 2, p, 3, o, 2, o, 3, 1) == -1  # ldc<N
    assert lib.oracle_gemm_f64(2, 2, 2, p, 2, p, 2, o, 2, None, 0, 1) == 0


# Planted mistakes: each rewrites one spot of oracle.c the way a plausible
# slip would (a dropped term, a transposed operand, a wrong index, a lost
# absolute value, a wrong sign, a stale accumulator).  At least one pin must
# fail for every mutant, or the pins would not pin the oracle.
MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < K; ++k)",
                    "for (int64_t k = 0; k + 1 < K; ++k)"),
    "drop_first_k": ("for (int64_t k = 0; k < K; ++k)",
                     "for (int64_t k = (K > 1); k < K; ++k)"),
    "b_transposed": ("const float *b = B + k * ldb;",
                     "const float *b = B + k;"),
    "a_row_stride": ("(double)A[i * lda + k]", "(double)A[i * K + k]"),
    "b_col_index": ("c[j] += a * (double)b[j];",
                    "c[j] += a * (double)b[j ? j - 1 : 0];"),
    "t_signed": ("t[j] += abs_a * fabs((double)b[j]);",
                 "t[j] += abs_a * (double)b[j];"),
    "c_sign": ("c[j] += a * (double)b[j];", "c[j] -= a * (double)b[j];"),
    "c_not_zeroed": ("for (int64_t j = 0; j < N; ++j) c[j] = 0.0;",
                     "for (int64_t j = 1; j < N; ++j) c[j] = 0.0;"),
    "float_accumulate": ("c[j] += a * (double)b[j];",
                         "c[j] = (float)(c[j] + (float)(a * (double)b[j]));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new, 1)
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src)
    so = str(tmp_path / f"liboracle_{name}.so")
    oracle_build.compile_source(str(path), so)
    lib = oracle.load_library(so)

    def gemm(A, B, **kw):
        return oracle.gemm(A, B, lib=lib, **kw)

    failed = []
    for pin in ALL_PINS:
        try:
            pin(gemm)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"


@pytest.mark.parametrize("pin", TRANSPOSE_PINS, ids=lambda p: p.__name__)
def test_transpose_pin(oracle_mod, pin):
    pin(oracle_mod.transpose)


# Every mutant keeps its accesses inside the buffers the wrapper allocates, so
# that a planted mistake fails a pin instead of corrupting the test process.
TRANSPOSE_MUTANTS = {
    "output_stride": ("out[j * ldo + i] = in[i * ldi + j];",
                      "out[j * rows + i] = in[i * ldi + j];"),
    "input_stride": ("out[j * ldo + i] = in[i * ldi + j];",
                     "out[j * ldo + i] = in[i * cols + j];"),
    "last_row_dropped": ("for (int64_t i = 0; i < rows; ++i)\n        for (int64_t j = 0; j < cols; ++j)",
                         "for (int64_t i = 0; i + 1 < rows; ++i)\n        for (int64_t j = 0; j < cols; ++j)"),
}


@pytest.mark.parametrize("name", sorted(TRANSPOSE_MUTANTS))
def test_transpose_pins_catch_planted_mistake(tmp_path, name):
    old, new = TRANSPOSE_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new, 1))
    so = str(tmp_path / f"liboracle_{name}.so")
    oracle_build.compile_source(str(path), so)
    lib = oracle.load_library(so)
    failed = []
    for pin in TRANSPOSE_PINS:
        try:
            pin(lambda A, **kw: oracle.transpose(A, lib=lib, **kw))
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
