/*
 * oracle.c -- CPU reference for the single-precision matrix product C = A·B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source with the HIP library.
 *
 * What it computes.  The pages describe tiling, shared-memory layouts,
 * vectorised loads and register tiles as changes to how data moves, not to
 * what is computed: the result is the textbook product ("CUDA in depth (5):
 * vectorized load and shared-memory layout", closing section on the GEMM data
 * path).  Storage is row-major with leading dimensions lda, ldb, ldc fixing
 * each row's start (same page, section on leading dimensions).  So, for
 * 0 <= i < M and 0 <= j < N:
 *
 *      C[i][j] = sum_{k=0}^{K-1} A[i*lda + k] * B[k*ldb + j]
 *      T[i][j] = sum_{k=0}^{K-1} |A[i*lda + k]| * |B[k*ldb + j]|
 *
 * T is the magnitude sum that scales the acceptance tolerance
 * |C_gpu - C| <= 1e-5 * T.
 *
 * How.  The plain triple loop, i outer, k middle, j inner, accumulating in
 * double.  Every product of two floats is exact in double (24 + 24 <= 53
 * significand bits), so each element's sum is formed strictly in increasing
 * k and the only rounding is that of the K-1 double additions.  Rows are
 * independent; they are shared among OpenMP threads, which does not change
 * any element's order of operations.  Compile without -ffast-math.
 *
 * Degenerate shapes: K == 0 gives C = T = 0 (the empty sum); M == 0 or N == 0
 * touches nothing.
 *
 * The file also holds the reference for the pages' tiled transpose kernel
 * ("Memory-bank mechanism and accelerated compute", section on the transpose
 * kernel): out[j][i] = in[i][j], a plain double loop.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the oracle would use by default (OMP_NUM_THREADS or all cores). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * C (M x N, leading dimension ldc) and, when T is not NULL, T (M x N, leading
 * dimension ldt) from A (M x K, lda) and B (K x N, ldb).  nthreads <= 0 means
 * the OpenMP default.  Returns 0, or -1 on a negative size or a leading
 * dimension smaller than the row it must hold.
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    double *C, int64_t ldc,
                    double *T, int64_t ldt,
                    int nthreads)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (lda < K || ldb < N || ldc < N || (T && ldt < N)) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif

#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        double *t = T ? T + i * ldt : NULL;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (t)
            for (int64_t j = 0; j < N; ++j) t[j] = 0.0;

        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                c[j] += a * (double)b[j];
            if (t) {
                const double abs_a = fabs(a);
                for (int64_t j = 0; j < N; ++j)
                    t[j] += abs_a * fabs((double)b[j]);
            }
        }
    }
    return 0;
}

/*
 * out (cols x rows, leading dimension ldo) = in^T, in being rows x cols with
 * leading dimension ldi: out[j*ldo + i] = in[i*ldi + j].  Gap columns of out
 * are not written.  Returns 0, or -1 on a negative size or a leading
 * dimension smaller than its row.
 */
int oracle_transpose_f32(int64_t rows, int64_t cols,
                         const float *in, int64_t ldi,
                         float *out, int64_t ldo)
{
    if (rows < 0 || cols < 0 || ldi < cols || ldo < rows) return -1;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            out[j * ldo + i] = in[i * ldi + j];
    return 0;
}
