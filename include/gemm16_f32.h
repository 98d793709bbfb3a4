/*
 * gemm16_f32.h -- GEMM with 16-bit inputs and FP32 accumulation on AMD
 * Instinct MI355X (gfx950), part of libsgemm_f32.so.
 *
 * A separate contract from sgemm_f32: the pages end on matrix units that take
 * 16-bit inputs and accumulate in FP32 ("Writing a Fast Matmul in CUDA, Step by
 * Step", section "Why LLMs use tensor cores instead"; "CUDA Matrix
 * Multiplication Optimization: From Naive to Near-cuBLAS", its list of lessons,
 * which ends on dedicated matrix hardware and 16-bit inputs).  It is not a
 * substitute for the FP32 product.
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * A and B hold 16-bit values (bfloat16 or IEEE binary16, one format for both,
 * given by in_type) as raw 16-bit patterns; C, alpha and beta are FP32.  op(),
 * the shapes, the row-major layout with leading dimensions in elements, the
 * transpose flags and the special cases (M == 0 or N == 0: nothing; alpha == 0
 * or K == 0: C = beta * C without reading A or B; beta == 0: C not read) are
 * those of sgemm_f32_ex in sgemm_f32.h.
 *
 * Arithmetic: the products of two 16-bit values are exact in FP32 and are
 * accumulated in FP32 on the matrix cores, so results agree with a float64
 * evaluation on the same 16-bit inputs to within
 * 2e-5 * (|alpha| * (|op(A)|*|op(B)|)_ij + |beta| * |C_ij|), and are exact when
 * every partial sum is (small integers).  The inputs are not rounded by the
 * library: rounding FP32 data to 16 bits is the caller's step.
 *
 * Layout and memory: the kernel reads both operands along K.  With trans_b == 1
 * (B stored N x K) and trans_a == 0, 16-byte aligned operands, row strides that
 * are multiples of 8 elements and K a multiple of 64, A and B are read in
 * place.  Otherwise the operands that do not meet this are first copied into a
 * K-major, zero-padded form in the call's scratch, taken as sgemm_f32.h
 * describes ((M or N) * K rounded up to 64 elements * 2 bytes each), which
 * costs one extra pass over them.  An operand given along M or N, A
 * transposed (trans_a == 1, K x M) or B as given (trans_b == 0, K x N), is
 * read in place too when it is aligned as above, its M or N is a multiple of
 * 8 and ldc is below about 2.1 million (256 rows of C addressable with 32-bit
 * byte offsets).  Grids of fewer than 128 tiles of 128 x 128 (small M or N)
 * split K over work-groups: their FP32 partial products, splits x M x N
 * floats, take scratch the same way, and a second kernel adds them in split
 * order and applies alpha and beta.
 *
 * Ownership and execution: device pointers owned by the caller, asynchronous on
 * `stream`, no synchronisation, thread-safe; as sgemm_f32.
 *
 * Return value: the codes of sgemm_f32_ex (0; 1, 2, 3; 5, 6, 7, 8, 10, 11; 22 when
 * K > 4000000 or the tile grid exceeds the launch limits; 23 for a transpose flag
 * other than 0 or 1; -(hipError_t)), and
 *     GEMM16_F32_ERR_TYPE           in_type is not GEMM16_F32_BF16 or GEMM16_F32_F16
 *     GEMM16_F32_ERR_ALIGN          A or B is not 2-byte aligned
 */
#ifndef GEMM16_F32_H
#define GEMM16_F32_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM16_F32_BF16 1
#define GEMM16_F32_F16 2
#define GEMM16_F32_ERR_ALIGN 21
#define GEMM16_F32_ERR_TYPE 25

int gemm16_f32(int in_type, int trans_a, int trans_b, int M, int N, int K, float alpha,
               const void *A, int lda, const void *B, int ldb,
               float beta, float *C, int ldc, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM16_F32_H */
