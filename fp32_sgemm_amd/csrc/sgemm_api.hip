// C interface: argument checks, special cases and kernel selection.
//
// The request is the BLAS-style single-precision GEMM C = alpha*A*B + beta*C on
// row-major matrices ("Learn: Optimizing GEMM", section 3; "How a Matmul Kernel
// Gets Fast", section 1).  A vendor library picks among many shape-specialised
// kernels ("Learn: Optimizing GEMM", section 8; "Writing a Fast Matmul in CUDA,
// Step by Step", section "In the real world"); this library picks among its own
// few kernels by shape and operand alignment, on the host, before one launch.
#include <cstdint>

#include "gemm_internal.hpp"
#include "sgemm_f32.h"

namespace {

using sgemm::GemmArgs;

int validate(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             const float *C, int ldc) {
    if (M < 0) return 1;
    if (N < 0) return 2;
    if (K < 0) return 3;
    const bool need_ab = M > 0 && N > 0 && K > 0 && alpha != 0.f;
    const bool need_c = M > 0 && N > 0;
    if (need_ab && A == nullptr) return 5;
    if (lda < (K > 1 ? K : 1)) return 6;
    if (need_ab && B == nullptr) return 7;
    if (ldb < (N > 1 ? N : 1)) return 8;
    if (need_c && C == nullptr) return 10;
    if (ldc < (N > 1 ? N : 1)) return 11;
    return 0;
}

// The 16-byte-load kernels need 16-byte aligned operands with row strides that
// are multiples of 4 floats, and address one slice of a tile with 32-bit byte
// offsets: 128 rows of A and 32 rows of B must span less than 2 GiB.
bool vec_aligned(const float *A, int lda, const float *B, int ldb) {
    const bool aligned = (reinterpret_cast<uintptr_t>(A) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(B) % 16 == 0) && (lda % 4 == 0) && (ldb % 4 == 0);
    const int64_t limit = (int64_t)1 << 31;
    const bool offsets_fit = (int64_t)(127 * (int64_t)lda + 32) * 4 < limit &&
                             (int64_t)(31 * (int64_t)ldb + 128) * 4 < limit;
    return aligned && offsets_fit;
}

// Large 128x128 tiles unless they leave most compute units idle and the
// 64x64 tiles give at least one tile per compute unit of the 256.
bool prefer_small_tiles(int M, int N) {
    const int64_t large = sgemm::mfma_large_grid(M, N);
    return large < 256;
}

bool aligned16(const float *A, int lda, const float *B, int ldb) {
    return (reinterpret_cast<uintptr_t>(A) % 16 == 0) && (reinterpret_cast<uintptr_t>(B) % 16 == 0) &&
           (lda % 4 == 0) && (ldb % 4 == 0);
}

int auto_variant(int M, int N, const float *A, int lda, const float *B, int ldb) {
    if (M <= sgemm::kSkinnyMaxM && sgemm::skinny_fits(lda, ldb)) return SGEMM_F32_SKINNY;
    if (!vec_aligned(A, lda, B, ldb)) return SGEMM_F32_MFMA_SCALAR;
    return prefer_small_tiles(M, N) ? SGEMM_F32_MFMA_SMALL : SGEMM_F32_MFMA_LARGE;
}

int to_status(hipError_t e) { return e == hipSuccess ? 0 : -static_cast<int>(e); }

constexpr int64_t kMaxGrid = 0x7fffffff;

int run(int variant, int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
        float beta, float *C, int ldc, hipStream_t stream) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    const int bad = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (bad) return bad;
    if (M == 0 || N == 0) return 0;

    GemmArgs g;
    g.M = M; g.N = N; g.K = K;
    g.alpha = alpha; g.beta = beta;
    g.A = A; g.B = B; g.C = C;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc;

    if (alpha == 0.f || K == 0) {
        if ((int64_t)M * N > (int64_t)1 << 62) return SGEMM_F32_ERR_TOO_LARGE;
        return to_status(sgemm::launch_scale_c(g, stream));
    }

    if (variant == SGEMM_F32_AUTO) variant = auto_variant(M, N, A, lda, B, ldb);
    const bool vec = vec_aligned(A, lda, B, ldb);
    switch (variant) {
        case SGEMM_F32_MFMA_LARGE:
            if (!vec) return SGEMM_F32_ERR_NOT_APPLICABLE;
            if (sgemm::mfma_large_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_mfma_large(g, true, stream));
        case SGEMM_F32_MFMA_SMALL:
            if (!vec) return SGEMM_F32_ERR_NOT_APPLICABLE;
            if (sgemm::mfma_small_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_mfma_small(g, true, stream));
        case SGEMM_F32_MFMA_SCALAR:
            if (prefer_small_tiles(M, N)) {
                if (sgemm::mfma_small_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
                return to_status(sgemm::launch_mfma_small(g, false, stream));
            }
            if (sgemm::mfma_large_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_mfma_large(g, false, stream));
        case SGEMM_F32_VALU:
            if (sgemm::valu_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_valu(g, vec, stream));
        case SGEMM_F32_SKINNY:
            if (M > sgemm::kSkinnyMaxM || !sgemm::skinny_fits(lda, ldb)) return SGEMM_F32_ERR_NOT_APPLICABLE;
            if (sgemm::skinny_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_skinny(g, aligned16(A, lda, B, ldb), stream));
        default:
            return SGEMM_F32_ERR_VARIANT;
    }
}

}  // namespace

extern "C" {

int sgemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
              float beta, float *C, int ldc, hipStream_t stream) {
    return run(SGEMM_F32_AUTO, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_variant(int variant, int M, int N, int K, float alpha, const float *A, int lda,
                      const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_select(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                     int ldb) {
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.f) return 0;
    return auto_variant(M, N, A, lda, B, ldb);
}

const char *sgemm_f32_variant_name(int variant) {
    switch (variant) {
        case SGEMM_F32_AUTO: return "auto";
        case SGEMM_F32_MFMA_LARGE: return "mfma_large";
        case SGEMM_F32_MFMA_SMALL: return "mfma_small";
        case SGEMM_F32_VALU: return "valu";
        case SGEMM_F32_SKINNY: return "skinny";
        case SGEMM_F32_MFMA_SCALAR: return "mfma_scalar";
        default: return nullptr;
    }
}

int sgemm_f32_version(void) { return 100; }

}  // extern "C"
