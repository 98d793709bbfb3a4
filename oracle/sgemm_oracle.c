/*
 * sgemm_oracle.c -- plain CPU reference for row-major single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header or constant with the
 * GPU library, and the GPU library never calls it.
 *
 * What it computes (the plain definition, nothing faster):
 *
 *   C = alpha * (A * B) + beta * C0
 *
 * with A an M x K matrix, B a K x N matrix and C0, C M x N matrices, all stored
 * row-major ("Learn: Optimizing GEMM", section 3 "Rung 0 -- Naive (recap)": the
 * listing's header comment states the operation and the three row-major shapes;
 * "How a Matmul Kernel Gets Fast", section 1 "The problem, and what cuBLAS is":
 * the two scalars scale the product and the existing C).  Element (i, j) is one
 * length-K dot product of row i of A with column j of B ("How a Matmul Kernel
 * Gets Fast", section 8 "Kernel 4: 1D blocktiling", which writes C[i][j] as the
 * sum over k of A[i][k] * B[k][j]).  The pages verify a GPU result against a
 * float64 dot product computed on the CPU ("Writing a Fast Matmul in CUDA, Step
 * by Step", section "Step 1: the problem and the yardstick"), so every sum here
 * is accumulated in double precision.
 *
 * Element addressing follows the row-major rule "base + row * stride + col"
 * ("CUDA Matrix Multiplication Optimization: From Naive to Near-cuBLAS", section
 * "Why Naive is Cache-Hostile"), with the stride of each matrix passed in
 * explicitly (lda, ldb, ldc) instead of being fixed to K and N.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - beta == 0: C0 is not read at all (so an uninitialised or NaN-filled C0
 *     gives a finite result), the usual BLAS convention.  Nothing is added in
 *     its place: the result is alpha * sum as it stands, so an exactly zero
 *     sum times a negative alpha is -0.0 (adding +0.0 would turn it into
 *     +0.0).
 *   - alpha == 0 or K == 0: there is no product term and A, B are not read;
 *     the result is beta * C0 alone (-0.0 where beta < 0 and C0 is +0.0), or
 *     +0.0 when beta == 0 as well.
 *   - Per element the products are added in the order k = 0, 1, ..., K-1.
 *     The product of two floats converted to double is exact (24 + 24 < 53
 *     significand bits), so whether the compiler fuses multiply and add does
 *     not change the accumulated value.
 *
 * Alongside C the oracle returns |A|*|B| (the sum over k of |A[i][k]*B[k][j]|),
 * which scales the element-wise error bound that real-valued results are held
 * to.
 */
#include <math.h>
#include <stdlib.h>
#include <omp.h>

/*
 * One element of the result from its two terms, with the special cases above:
 * the old value C0[at] is read only when beta != 0, and a term that is absent is
 * not added as a zero.
 */
static double combine(int use_product, double alpha, double acc, float beta,
                      const float *C0, long at)
{
    if (beta == 0.0f)
        return use_product ? alpha * acc : 0.0;
    const double old = (double)beta * (double)C0[at];
    return use_product ? alpha * acc + old : old;
}

/* Number of OpenMP threads the full-matrix routine will use. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Sets that number (n >= 1; used to time the oracle on a single core). */
void oracle_set_num_threads(int n) {
    if (n >= 1) omp_set_num_threads(n);
}

/*
 * Full product.  Cref and absab (absab may be NULL) are M x N row-major double
 * arrays with row stride N.  Returns 0 on success, -1 if scratch memory could
 * not be allocated, 1 on a negative size.
 */
int oracle_sgemm_f64(int M, int N, int K, float alpha,
                     const float *A, long lda,
                     const float *B, long ldb,
                     float beta, const float *C0, long ldc,
                     double *Cref, double *absab)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (M == 0 || N == 0) return 0;
    const int use_product = (alpha != 0.0f) && (K > 0);
    const double a_s = (double)alpha;
    int failed = 0;

#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        double *aac = (double *)malloc(sizeof(double) * (size_t)N);
        if (acc == NULL || aac == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < M; ++i) {
            if (acc == NULL || aac == NULL) continue;
            for (int j = 0; j < N; ++j) { acc[j] = 0.0; aac[j] = 0.0; }
            if (use_product) {
                for (int k = 0; k < K; ++k) {
                    const double a = (double)A[(long)i * lda + k];
                    const float *brow = B + (long)k * ldb;
                    for (int j = 0; j < N; ++j) {
                        const double p = a * (double)brow[j];
                        acc[j] += p;
                        aac[j] += fabs(p);
                    }
                }
            }
            for (int j = 0; j < N; ++j) {
                Cref[(long)i * N + j] = combine(use_product, a_s, acc[j], beta, C0,
                                                (long)i * ldc + j);
                if (absab != NULL) absab[(long)i * N + j] = use_product ? aac[j] : 0.0;
            }
        }
        free(acc);
        free(aac);
    }
    return failed ? -1 : 0;
}

/*
 * Selected entries only: for t in [0, n) computes element (rows[t], cols[t]) of
 * the same product, with the same k order, into out[t] (and absab[t] when
 * absab is not NULL).  Used to check results of products too large to form in
 * full on the CPU.  Returns 1 if an index is out of range.
 */
int oracle_sgemm_f64_entries(int M, int N, int K, float alpha,
                             const float *A, long lda,
                             const float *B, long ldb,
                             float beta, const float *C0, long ldc,
                             long n, const long *rows, const long *cols,
                             double *out, double *absab)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    for (long t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return 1;
    const int use_product = (alpha != 0.0f) && (K > 0);

#pragma omp parallel for schedule(static)
    for (long t = 0; t < n; ++t) {
        const long i = rows[t], j = cols[t];
        double acc = 0.0, aac = 0.0;
        if (use_product) {
            for (int k = 0; k < K; ++k) {
                const double p = (double)A[i * lda + k] * (double)B[(long)k * ldb + j];
                acc += p;
                aac += fabs(p);
            }
        }
        out[t] = combine(use_product, (double)alpha, acc, beta, C0, i * ldc + j);
        if (absab != NULL) absab[t] = use_product ? aac : 0.0;
    }
    return 0;
}

/*
 * Transposed operands.  The library the pages compare against handles every
 * transpose of its operands, and its kernel names carry the operand forms
 * ("nn": neither operand transposed) ("Writing a Fast Matmul in CUDA, Step by
 * Step", section "In the real world").  Here op(A) is the M x K left operand
 * and op(B) the K x N right operand of the same product:
 *
 *   trans_a == 0:  A is stored M x K and op(A)(i, k) = A[i*lda + k]
 *   trans_a != 0:  A is stored K x M and op(A)(i, k) = A[k*lda + i]
 *   trans_b == 0:  B is stored K x N and op(B)(k, j) = B[k*ldb + j]
 *   trans_b != 0:  B is stored N x K and op(B)(k, j) = B[j*ldb + k]
 *
 * C = alpha * op(A) * op(B) + beta * C0, with C0 and C M x N row-major as
 * above, the same special cases, and the same k order.  Written element by
 * element through op_elem, with no reordering for speed.
 */
static double op_elem(const float *X, long ld, int trans, long r, long c)
{
    return (double)(trans ? X[c * ld + r] : X[r * ld + c]);
}

static void op_dot(int trans_a, int trans_b, int K, const float *A, long lda,
                   const float *B, long ldb, long i, long j,
                   double *acc_out, double *aac_out)
{
    double acc = 0.0, aac = 0.0;
    for (int k = 0; k < K; ++k) {
        const double p = op_elem(A, lda, trans_a, i, k) * op_elem(B, ldb, trans_b, k, j);
        acc += p;
        aac += fabs(p);
    }
    *acc_out = acc;
    *aac_out = aac;
}

/* Full product with transposed operands; Cref and absab as in oracle_sgemm_f64. */
int oracle_sgemm_op_f64(int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const float *A, long lda,
                        const float *B, long ldb,
                        float beta, const float *C0, long ldc,
                        double *Cref, double *absab)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (M == 0 || N == 0) return 0;
    const int use_product = (alpha != 0.0f) && (K > 0);

#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
        for (int j = 0; j < N; ++j) {
            double acc = 0.0, aac = 0.0;
            if (use_product) op_dot(trans_a, trans_b, K, A, lda, B, ldb, i, j, &acc, &aac);
            Cref[(long)i * N + j] = combine(use_product, (double)alpha, acc, beta, C0,
                                            (long)i * ldc + j);
            if (absab != NULL) absab[(long)i * N + j] = use_product ? aac : 0.0;
        }
    }
    return 0;
}

/* Selected entries of the product with transposed operands. */
int oracle_sgemm_op_f64_entries(int trans_a, int trans_b, int M, int N, int K, float alpha,
                                const float *A, long lda,
                                const float *B, long ldb,
                                float beta, const float *C0, long ldc,
                                long n, const long *rows, const long *cols,
                                double *out, double *absab)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    for (long t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return 1;
    const int use_product = (alpha != 0.0f) && (K > 0);

#pragma omp parallel for schedule(static)
    for (long t = 0; t < n; ++t) {
        const long i = rows[t], j = cols[t];
        double acc = 0.0, aac = 0.0;
        if (use_product) op_dot(trans_a, trans_b, K, A, lda, B, ldb, i, j, &acc, &aac);
        out[t] = combine(use_product, (double)alpha, acc, beta, C0, i * ldc + j);
        if (absab != NULL) absab[t] = use_product ? aac : 0.0;
    }
    return 0;
}

/*
 * 16-bit input formats for the lower-precision form of the product (the pages'
 * endpoint: matrix units that take 16-bit inputs and accumulate in FP32, "CUDA
 * Matrix Multiplication Optimization: From Naive to Near-cuBLAS", its list of
 * lessons, which ends on dedicated matrix hardware and 16-bit inputs; "Writing
 * a Fast Matmul in CUDA, Step by Step", section "Why LLMs use tensor cores
 * instead").  Decoded here from the field layouts of the formats, value by
 * value, into float (every value of either format is exactly a float):
 *
 *   bfloat16: sign (1 bit), exponent (8, bias 127), fraction (7)
 *   binary16: sign (1 bit), exponent (5, bias 15),  fraction (10)
 *
 * exponent 0 is zero or subnormal (2^(1-bias) * fraction / 2^bits), all ones
 * is infinity (fraction 0) or NaN.  The product then is the float64 oracle
 * above on the decoded matrices: the decoded values are exact, so the
 * reference carries no rounding of the inputs.
 */
static float decode_16(unsigned v, int exp_bits, int frac_bits, int bias)
{
    const unsigned sign = v >> (exp_bits + frac_bits);
    const unsigned e = (v >> frac_bits) & ((1u << exp_bits) - 1u);
    const unsigned f = v & ((1u << frac_bits) - 1u);
    const double scale = (double)(1u << frac_bits);
    double x;
    if (e == (1u << exp_bits) - 1u)
        x = f ? NAN : INFINITY;
    else if (e == 0)
        x = ldexp((double)f / scale, 1 - bias);
    else
        x = ldexp(1.0 + (double)f / scale, (int)e - bias);
    return (float)(sign ? -x : x);
}

/* kind 1: bfloat16, kind 2: binary16.  Returns 1 for another kind. */
int oracle_decode_16(int kind, const unsigned short *in, long n, float *out)
{
    if (kind != 1 && kind != 2) return 1;
    for (long t = 0; t < n; ++t)
        out[t] = kind == 1 ? decode_16(in[t], 8, 7, 127) : decode_16(in[t], 5, 10, 15);
    return 0;
}
