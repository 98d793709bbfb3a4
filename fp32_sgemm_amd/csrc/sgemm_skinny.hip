// FP32 GEMM for M <= 16 (a short, wide A times a tall B), on 16x16x4 MFMA.
//
// With M = 16 and N = K = 4096 the product does 8 FLOP per byte of B it must
// stream, below the MI355X ridge point of about 20 FLOP per byte, so the kernel
// is bound by HBM bandwidth: its job is to stream B exactly once with enough
// loads in flight.  (Decode-time GEMV-like shapes sit on the bandwidth roof,
// "Writing a Fast Matmul in CUDA, Step by Step", section "In the real world";
// too few output tiles to fill the machine is the case where the reduction is
// split, "How a Matmul Kernel Gets Fast", section 15.)
//
// Each work-group owns a 16-column strip of C and all M <= 16 rows.  Its NW
// waves split K into contiguous ranges; each wave streams its rows of the strip
// straight from global memory into MFMA operand registers (no LDS staging: no
// element of B is used by more than one wave).  For a group of 16 k values a
// lane loads A(l % 16, k0 + 4*(l/16) + 0..3) as one 16-byte load and the four
// B values B(k0 + 4*(l/16) + e, n0 + l % 16), e = 0..3, then issues four
// v_mfma_f32_16x16x4_f32 in which lane l supplies k = k0 + 4*(l/16) + e.  The
// per-wave partial 16x16 tiles are added in LDS in a fixed wave order, so the
// result does not depend on timing.
#include "gemm_internal.hpp"

namespace sgemm {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int SK_NW = 8;                 // waves per work-group
constexpr int SK_NT = SK_NW * 64;
constexpr int SK_BN = 16;                // columns of C per work-group
constexpr int SK_UNROLL = 8;             // 16-row groups in flight per wave

__device__ __forceinline__ void skinny_group(const GemmArgs &g, int n0, int kg, int lane,
                                             bool guard, f32x4v &acc) {
    const int i = lane & 15;                       // row of A / column of the strip
    const int kq = kg + 4 * (lane >> 4);           // first of this lane's 4 k values
    float a[4], b[4];
    if (!guard) {
        const float *pa = g.A + (int64_t)i * g.lda + kq;
        a[0] = pa[0]; a[1] = pa[1]; a[2] = pa[2]; a[3] = pa[3];
        const float *pb = g.B + (int64_t)kq * g.ldb + n0 + i;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = pb[e * g.ldb];
    } else {
        const bool rin = i < g.M, cin = n0 + i < g.N;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool kin = kq + e < g.K;
            a[e] = (rin && kin) ? g.A[(int64_t)i * g.lda + kq + e] : 0.f;
            b[e] = (cin && kin) ? g.B[(int64_t)(kq + e) * g.ldb + n0 + i] : 0.f;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
}

__global__ __launch_bounds__(SK_NT) void sgemm_skinny_kernel(GemmArgs g, int tiles_n) {
    __shared__ float red[SK_NW][16 * 16];
    int tm, tn;
    tile_of_block(blockIdx.x, 1, tiles_n, 1, tm, tn);
    const int n0 = tn * SK_BN;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // Contiguous K range of this wave, in whole groups of 16.
    const int groups = (g.K + 15) / 16;
    const int per_wave = (groups + SK_NW - 1) / SK_NW;
    const int gbeg = wave * per_wave;
    const int gend = min(groups, gbeg + per_wave);
    const bool edge = (g.M < 16) || (n0 + SK_BN > g.N);

    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
    int gi = gbeg;
    for (; gi + SK_UNROLL <= gend; gi += SK_UNROLL) {
        const bool guard = edge || (gi + SK_UNROLL) * 16 > g.K;
#pragma unroll
        for (int u = 0; u < SK_UNROLL; ++u) skinny_group(g, n0, (gi + u) * 16, lane, guard, acc);
    }
    for (; gi < gend; ++gi) skinny_group(g, n0, gi * 16, lane, true, acc);

    // Accumulator register r holds row 4*(l/16) + r, column l % 16.
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < SK_NW; ++w) s += red[w][threadIdx.x];
        if (row < g.M && n0 + col < g.N) {
            float *p = g.C + (int64_t)row * g.ldc + n0 + col;
            float v = g.alpha * s;
            if (g.beta != 0.f) v = fmaf(g.beta, *p, v);
            *p = v;
        }
    }
}

}  // namespace

int64_t skinny_grid(int M, int N) {
    (void)M;
    return (N + SK_BN - 1) / SK_BN;
}

hipError_t launch_skinny(const GemmArgs &g, hipStream_t stream) {
    const int tiles_n = (g.N + SK_BN - 1) / SK_BN;
    hipLaunchKernelGGL(sgemm_skinny_kernel, dim3(tiles_n), dim3(SK_NT), 0, stream, g, tiles_n);
    return hipGetLastError();
}

}  // namespace sgemm
