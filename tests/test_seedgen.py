"""The seeded input generator (CPU only)."""
import numpy as np

import seedgen


def test_splitmix64_published_vectors():
    # First outputs of SplitMix64 started from state 0, as printed with the
    # generator's public reference implementation.
    got = seedgen.splitmix64(0, 0, 3)
    assert [int(v) for v in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                     0x06C45D188009454F]


def test_counter_form_is_position_independent():
    whole = seedgen.draw("uniform", 7, 0, 5000)
    part = seedgen.draw("uniform", 7, 1234, 100)
    assert np.array_equal(whole[1234:1334], part)
    big = seedgen.draw("normal", 3, 0, (1 << 20) + 17)   # spans two chunks
    assert np.array_equal(big[(1 << 20) - 5:], seedgen.draw("normal", 3, (1 << 20) - 5, 22))


def test_uniform_grid_and_range():
    v = seedgen.draw("uniform", 2, 0, 1 << 18).astype(np.float64)
    assert v.min() >= -1.0 and v.max() < 1.0
    m = (v + 1.0) * 2.0 ** 23          # integers on the 2**-23 grid
    assert np.array_equal(m, np.round(m))
    assert abs(v.mean()) < 0.01 and abs(v.var() - 1.0 / 3.0) < 0.01


def test_normal_moments():
    v = seedgen.draw("normal", 4, 0, 1 << 18).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    assert np.all(np.isfinite(v))


def test_gemm_inputs_layout():
    A, B = seedgen.gemm_inputs(3, 5, 4, "uniform", 9, lda=6, ldb=7, fill=-7.0)
    assert A.shape == (3, 6) and B.shape == (4, 7)
    assert np.all(A[:, 4:] == -7.0) and np.all(B[:, 5:] == -7.0)
    flat = seedgen.draw("uniform", 9, 0, 3 * 4 + 4 * 5)
    assert np.array_equal(A[:, :4].ravel(), flat[:12])
    assert np.array_equal(B[:, :5].ravel(), flat[12:])


def test_integer_matrix_bounds():
    x = seedgen.integer_matrix(50, 60, -8, 8, 5)
    assert x.min() == -8 and x.max() == 8
    assert np.array_equal(x, np.round(x))
