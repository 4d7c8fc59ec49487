/*
 * CPU oracle for row-major FP32 matrix multiplication, C = A x B.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It shares
 * no source, header or helper with the GPU path and includes no HIP header.
 *
 * What it computes (the plain definition, nothing more):
 *
 *   C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 *
 *   - Each output cell is the dot product of row i of A with column j of B
 *     ("Tiled Matrix Multiplication in CUDA", section 1, "What matrix
 *     multiplication actually does"; "Tiled GEMM: Matrix Multiplication in
 *     CUDA", section 1, the definition of C[i, j]).
 *   - Matrices are stored row-major: cell (r, c) of a matrix with leading
 *     dimension ld sits at flat index r * ld + c ("Tiled Matrix Multiplication
 *     in CUDA", section 2, "flat indexing").  With ld equal to the row width
 *     this is exactly the pages' formula; a larger ld describes a row-major
 *     sub-matrix of a wider allocation.
 *   - Rectangular shapes follow "Tiled GEMM: Matrix Multiplication in CUDA",
 *     section 7.1 (ragged edges): A is M x K, B is K x N, C is M x N.
 *
 * Arithmetic (the pages keep a float accumulator; this oracle is the exact
 * reference the GPU result is judged against, so it accumulates in double):
 *   1. every FP32 operand is widened to FP64; the product of two widened
 *      floats is exact (24 + 24 significand bits fit in 53);
 *   2. the products are added into an FP64 accumulator in ascending k;
 *   3. the FP64 sum is rounded once to FP32 (round to nearest even, the C
 *      conversion under the default rounding mode).
 *   The FP64 sums are also returned on request, for error metrics.
 *
 * Loop order.  For one row i the code keeps one FP64 accumulator per output
 * column j and walks k in ascending order, adding A[i][k] * B[k][j] into
 * accumulator j.  Each accumulator therefore receives exactly the sequence
 * 0 + A[i][0]B[0][j] + A[i][1]B[1][j] + ... of the definition; only the
 * interleaving between different columns differs from an i-j-k nest, and the
 * columns never interact.  Rows are independent ("every cell of C is
 * independent", section 1 of the first page), so OpenMP splits the row range
 * across threads and the result is identical for any thread count.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 * Contraction is switched off although it would not change the result (an
 * exact product added once rounds the same fused or not).
 */

#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/*
 * One output row.  `a_row` is row i of A (K floats), B is K x N with leading
 * dimension ldb, `acc` is scratch of N doubles, `c32` receives N floats and
 * `c64` (may be NULL) N doubles.
 */
static void oracle_one_row(int64_t N, int64_t K, const float *a_row,
                           const float *B, int64_t ldb, double *acc,
                           float *c32, double *c64)
{
    for (int64_t j = 0; j < N; ++j)
        acc[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double a_ik = (double)a_row[k];
        const float *b_row = B + k * ldb;
        for (int64_t j = 0; j < N; ++j)
            acc[j] += a_ik * (double)b_row[j];
    }
    for (int64_t j = 0; j < N; ++j) {
        c32[j] = (float)acc[j];
        if (c64)
            c64[j] = acc[j];
    }
}

/*
 * Computes selected rows of C = A x B.
 *
 *   M, N, K    logical sizes (A is M x K, B is K x N), all >= 0
 *   A, lda     row-major A, lda >= K (unused when M == 0 or K == 0)
 *   B, ldb     row-major B, ldb >= N (unused when K == 0 or N == 0)
 *   rows       NULL for all rows 0..M-1 (then nrows must equal M), else a list
 *              of nrows row indices in [0, M)
 *   C, ldc     output, nrows x N with leading dimension ldc >= N; output row t
 *              holds row rows[t] of the product (row t when rows is NULL).
 *              Elements of C beyond column N - 1 are not written.
 *   C64, ldc64 optional FP64 sums in the same arrangement (NULL to skip)
 *   threads    OpenMP threads, <= 0 for the runtime default
 *
 * K == 0 gives rows of zeros (the empty sum).  Returns ORACLE_OK, or
 * ORACLE_EINVAL / ORACLE_ENOMEM without writing anything.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                const int64_t *rows, int64_t nrows,
                float *C, int64_t ldc,
                double *C64, int64_t ldc64,
                int threads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0)
        return ORACLE_EINVAL;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return ORACLE_EINVAL;
    if (C64 && ldc64 < (N > 1 ? N : 1))
        return ORACLE_EINVAL;
    if (rows == NULL && nrows != M)
        return ORACLE_EINVAL;
    if (rows != NULL) {
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= M)
                return ORACLE_EINVAL;
    }
    if (nrows == 0 || N == 0)
        return ORACLE_OK;
    if (C == NULL || (K > 0 && (A == NULL || B == NULL)))
        return ORACLE_EINVAL;

    int nthreads = 1;
#ifdef _OPENMP
    nthreads = threads > 0 ? threads : omp_get_max_threads();
#endif
    /* one accumulator row per thread, allocated before the parallel region */
    double *scratch = (double *)malloc((size_t)nthreads * (size_t)N * sizeof(double));
    if (scratch == NULL)
        return ORACLE_ENOMEM;

#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t t = 0; t < nrows; ++t) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        const int64_t i = rows ? rows[t] : t;
        const float *a_row = K > 0 ? A + i * lda : NULL;
        oracle_one_row(N, K, a_row, B, ldb, scratch + (size_t)tid * (size_t)N,
                       C + t * ldc, C64 ? C64 + t * ldc64 : NULL);
    }
    free(scratch);
    return ORACLE_OK;
}

/* Number of OpenMP threads a call with `threads` <= 0 would use. */
int oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
