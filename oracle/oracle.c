/*
 * CPU oracle for the dense GEMM  D = alpha * op(A) * op(B) + beta * C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The GPU product
 * path never links, loads or calls it, and shares no code with it.
 *
 * What it computes is the plain definition from "GEMM on NVIDIA GPUs: from a
 * naive kernel to a tiled pipeline", section 1:
 *     D_ij = alpha * sum_{k=0}^{K-1} op(A)_ik op(B)_kj + beta * C_ij
 * with op(X) either X or X transposed.  It also returns, for every requested
 * output, the error-bound denominator  sum_k |op(A)_ik| |op(B)_kj| + |beta C_ij|
 * that the parity check divides by.
 *
 * Precision: every input (fp32, or bf16 given as raw 16-bit patterns) is
 * widened to double exactly; each product of two such values is exact in
 * double (at most 48 significant bits); the K products are summed one after
 * another in increasing k, in double.  The relative rounding error of the sum
 * is therefore at most about K * 2^-53, far below the fp32 and bf16 parity
 * tolerances.  When beta == 0 the matrix C is never read (it may be NULL), so
 * NaN or Inf in C cannot reach the result; when K == 0 the sum is empty.
 *
 * Storage is row-major:
 *   transA == 0: A is M x K, element (i,k) at A[i*lda + k]
 *   transA == 1: A is K x M, element (i,k) of op(A) at A[k*lda + i]
 *   transB == 0: B is K x N, element (k,j) at B[k*ldb + j]
 *   transB == 1: B is N x K, element (k,j) of op(B) at B[j*ldb + k]
 *   C is M x N, element (i,j) at C[i*ldc + j]
 *
 * Built with gcc -O2 -ffp-contract=off (no fast-math), optionally OpenMP.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes: 0 = A,B are float (fp32); 1 = A,B are bfloat16 bit patterns. */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* bfloat16 is the upper half of an IEEE binary32: shift the 16 bits into the
 * high half and reinterpret.  Exact for every pattern (incl. NaN/Inf/subnormal). */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_operand(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/* op(A)_(i,k) */
static double opA(const void *A, int dtype, int transA, int64_t lda, int64_t i, int64_t k)
{
    return transA ? load_operand(A, dtype, k * lda + i)
                  : load_operand(A, dtype, i * lda + k);
}

/* op(B)_(k,j) */
static double opB(const void *B, int dtype, int transB, int64_t ldb, int64_t k, int64_t j)
{
    return transB ? load_operand(B, dtype, j * ldb + k)
                  : load_operand(B, dtype, k * ldb + j);
}

/*
 * Evaluate npts outputs (rows[p], cols[p]).
 * out_val[p] = alpha * s + beta * C_ij   (the beta term only when beta != 0)
 * out_den[p] = sum_k |a||b| + |beta * C_ij|
 * Returns 0 on success, -1 on an invalid argument.
 */
int oracle_gemm_points(int dtype, int transA, int transB,
                       int64_t M, int64_t N, int64_t K,
                       double alpha, const void *A, int64_t lda,
                       const void *B, int64_t ldb,
                       double beta, const float *C, int64_t ldc,
                       int64_t npts, const int64_t *rows, const int64_t *cols,
                       double *out_val, double *out_den, int nthreads)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || M < 0 || N < 0 || K < 0 || npts < 0)
        return -1;
    if (K > 0 && (A == 0 || B == 0))
        return -1;
    if (beta != 0.0 && C == 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t i = rows[p];
        const int64_t j = cols[p];
        double s = 0.0;
        double den = 0.0;
        if (i >= 0 && i < M && j >= 0 && j < N) {
            for (int64_t k = 0; k < K; ++k) {
                const double a = opA(A, dtype, transA, lda, i, k);
                const double b = opB(B, dtype, transB, ldb, k, j);
                s += a * b;
                den += fabs(a) * fabs(b);
            }
            double d = alpha * s;
            if (beta != 0.0) {
                const double c = (double)C[i * ldc + j];
                d += beta * c;
                den += fabs(beta * c);
            }
            out_val[p] = d;
            out_den[p] = den;
        } else {
            out_val[p] = NAN;
            out_den[p] = NAN;
        }
    }
    return 0;
}

/* Threads the OpenMP runtime would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
