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

int at_least_one(int v) { return v > 1 ? v : 1; }

// Row widths of the stored A and B: A is M x K (K x M when transposed), B is
// K x N (N x K when transposed).
int validate(int ta, int tb, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
             int ldb, const float *C, int ldc) {
    if (ta != 0 && ta != 1) return SGEMM_F32_ERR_TRANS;
    if (tb != 0 && tb != 1) return SGEMM_F32_ERR_TRANS;
    if (M < 0) return 1;
    if (N < 0) return 2;
    if (K < 0) return 3;
    const bool need_ab = M > 0 && N > 0 && K > 0 && alpha != 0.f;
    const bool need_c = M > 0 && N > 0;
    if (need_ab && A == nullptr) return 5;
    if (lda < at_least_one(ta ? M : K)) return 6;
    if (need_ab && B == nullptr) return 7;
    if (ldb < at_least_one(tb ? K : N)) return 8;
    if (need_c && C == nullptr) return 10;
    if (ldc < (N > 1 ? N : 1)) return 11;
    return 0;
}

// The 16-byte-load kernels need 16-byte aligned operands with row strides that
// are multiples of 4 floats, and address one slice of a tile with 32-bit byte
// offsets: the stored rows that one slice touches must span less than 2 GiB
// (128 rows for an operand read along k: A as given, B transposed; 32 rows for
// one read along M or N: B as given, A transposed).
bool slice_fits(bool k_major, int ld) {
    const int64_t limit = (int64_t)1 << 31;
    const int64_t span = k_major ? 127 * (int64_t)ld + 32 : 31 * (int64_t)ld + 128;
    return span * 4 < limit;
}

bool vec_aligned(int ta, int tb, const float *A, int lda, const float *B, int ldb) {
    const bool aligned = (reinterpret_cast<uintptr_t>(A) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(B) % 16 == 0) && (lda % 4 == 0) && (ldb % 4 == 0);
    return aligned && slice_fits(!ta, lda) && slice_fits(tb, ldb);
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

// Transposed operands go to the MFMA kernels only.
int auto_variant(int ta, int tb, int M, int N, const float *A, int lda, const float *B, int ldb) {
    if (!ta && !tb && M <= sgemm::kSkinnyMaxM && sgemm::skinny_fits(lda, ldb)) return SGEMM_F32_SKINNY;
    if (!vec_aligned(ta, tb, A, lda, B, ldb)) return SGEMM_F32_MFMA_SCALAR;
    return prefer_small_tiles(M, N) ? SGEMM_F32_MFMA_SMALL : SGEMM_F32_MFMA_LARGE;
}

int to_status(hipError_t e) { return e == hipSuccess ? 0 : -static_cast<int>(e); }

constexpr int64_t kMaxGrid = 0x7fffffff;

int run(int variant, int ta, int tb, int M, int N, int K, float alpha, const float *A, int lda,
        const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    const int bad = validate(ta, tb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (bad) return bad;
    if (M == 0 || N == 0) return 0;

    GemmArgs g;
    g.M = M; g.N = N; g.K = K;
    g.alpha = alpha; g.beta = beta;
    g.A = A; g.B = B; g.C = C;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc;
    g.trans_a = ta; g.trans_b = tb;

    if (alpha == 0.f || K == 0) {
        if ((int64_t)M * N > (int64_t)1 << 62) return SGEMM_F32_ERR_TOO_LARGE;
        return to_status(sgemm::launch_scale_c(g, stream));
    }

    if (variant == SGEMM_F32_AUTO) variant = auto_variant(ta, tb, M, N, A, lda, B, ldb);
    const bool vec = vec_aligned(ta, tb, A, lda, B, ldb);
    const bool plain = !ta && !tb;
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
            if (!plain) return SGEMM_F32_ERR_NOT_APPLICABLE;
            if (sgemm::valu_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_valu(g, vec, stream));
        case SGEMM_F32_SKINNY:
            if (!plain || M > sgemm::kSkinnyMaxM || !sgemm::skinny_fits(lda, ldb))
                return SGEMM_F32_ERR_NOT_APPLICABLE;
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
    return run(SGEMM_F32_AUTO, 0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_variant(int variant, int M, int N, int K, float alpha, const float *A, int lda,
                      const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(variant, 0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_select(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                     int ldb) {
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.f) return 0;
    return auto_variant(0, 0, M, N, A, lda, B, ldb);
}

int sgemm_f32_ex(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A, int lda,
                 const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(SGEMM_F32_AUTO, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_ex_variant(int variant, int trans_a, int trans_b, int M, int N, int K, float alpha,
                         const float *A, int lda, const float *B, int ldb, float beta, float *C, int ldc,
                         hipStream_t stream) {
    return run(variant, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_ex_select(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A, int lda,
                        const float *B, int ldb) {
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return 0;
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.f) return 0;
    return auto_variant(trans_a, trans_b, M, N, A, lda, B, ldb);
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

int sgemm_f32_version(void) { return 200; }

}  // extern "C"
