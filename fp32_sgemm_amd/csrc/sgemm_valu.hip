// FP32 GEMM on the vector ALUs: the comparison path for the matrix-core kernels.
//
// This is the register-blocked outer-product scheme of "Learn: Optimizing
// GEMM" section 6 ("Rung 3 & 4") and "How a Matmul Kernel Gets Fast" section 9:
// a 128x128 block tile, BK = 8, 256 threads, each thread accumulating an 8x8
// sub-tile in registers from 8 values of A and 8 values of B per k step.  The
// A slice is stored transposed in LDS (k-major, "Learn: Optimizing GEMM"
// section 7), so a thread's 8 A values are two 16-byte reads, as are its 8 B
// values.  Each thread's 8x8 tile is split into four 4x4 pieces 64 rows and 64
// columns apart ("Writing a Fast Matmul in CUDA, Step by Step", section "Bank
// conflicts and double buffering"), so the 16 threads of a row group read 16
// consecutive 16-byte B groups.  Two LDS buffers with register-staged prefetch
// give one barrier per slice.  The arithmetic is one v_fma_f32 per
// multiply-add (packed FP32 instructions are disabled at compile time).
#include "gemm_internal.hpp"

namespace sgemm {
namespace {

constexpr int VBM = 128, VBN = 128, VBK = 8, VNT = 256;
constexpr int VAS = VBM + 4;               // LDS row stride of the transposed A slice
constexpr int VA_STAGE = VBK * VAS;
constexpr int VB_STAGE = VBK * VBN;
constexpr int VSTAGE = VA_STAGE + VB_STAGE;

template <bool VEC, bool GUARD>
__device__ __forceinline__ float4 vload4(const float *__restrict__ base, int64_t ld, int row, int col,
                                         int rows, int cols) {
    const float *p = base + (int64_t)row * ld + col;
    if (!GUARD) {
        if (VEC) return *reinterpret_cast<const float4 *>(p);
        return make_float4(p[0], p[1], p[2], p[3]);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < rows) {
        if (VEC && col + 3 < cols) {
            v = *reinterpret_cast<const float4 *>(p);
        } else {
            if (col + 0 < cols) v.x = p[0];
            if (col + 1 < cols) v.y = p[1];
            if (col + 2 < cols) v.z = p[2];
            if (col + 3 < cols) v.w = p[3];
        }
    }
    return v;
}

template <bool VEC, bool GUARD>
__device__ __forceinline__ void vload_slice(const GemmArgs &g, int m0, int n0, int k0, int tid,
                                            float4 &ra, float4 &rb) {
    // A: 128 rows x 2 groups of 4 k; B: 8 rows x 32 groups of 4 n.
    ra = vload4<VEC, GUARD>(g.A, g.lda, m0 + (tid >> 1), k0 + (tid & 1) * 4, g.M, g.K);
    rb = vload4<VEC, GUARD>(g.B, g.ldb, k0 + (tid >> 5), n0 + (tid & 31) * 4, g.K, g.N);
}

__device__ __forceinline__ void vstore_slice(float *stage, int tid, const float4 &ra, const float4 &rb) {
    float *As = stage;
    const int m = tid >> 1, k = (tid & 1) * 4;
    As[(k + 0) * VAS + m] = ra.x;
    As[(k + 1) * VAS + m] = ra.y;
    As[(k + 2) * VAS + m] = ra.z;
    As[(k + 3) * VAS + m] = ra.w;
    *reinterpret_cast<float4 *>(stage + VA_STAGE + (tid >> 5) * VBN + (tid & 31) * 4) = rb;
}

template <bool VEC>
__global__ __launch_bounds__(VNT) void sgemm_valu_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    __shared__ __attribute__((aligned(16))) float smem[2 * VSTAGE];
    poison_lds<sizeof(smem)>(smem);
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * VBM, n0 = tn * VBN;
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    const bool edge_mn = (m0 + VBM > g.M) || (n0 + VBN > g.N);
    const int nk = (g.K + VBK - 1) / VBK;
    float4 ra, rb;
    if (edge_mn || VBK > g.K) vload_slice<VEC, true>(g, m0, n0, 0, tid, ra, rb);
    else vload_slice<VEC, false>(g, m0, n0, 0, tid, ra, rb);
    vstore_slice(smem, tid, ra, rb);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const bool more = t + 1 < nk;
        if (more) {
            const int k0 = (t + 1) * VBK;
            if (edge_mn || k0 + VBK > g.K) vload_slice<VEC, true>(g, m0, n0, k0, tid, ra, rb);
            else vload_slice<VEC, false>(g, m0, n0, k0, tid, ra, rb);
        }
        const float *As = smem + (t & 1) * VSTAGE;
        const float *Bs = As + VA_STAGE;
#pragma unroll
        for (int k = 0; k < VBK; ++k) {
            const float4 a0 = *reinterpret_cast<const float4 *>(As + k * VAS + ty * 4);
            const float4 a1 = *reinterpret_cast<const float4 *>(As + k * VAS + 64 + ty * 4);
            const float4 b0 = *reinterpret_cast<const float4 *>(Bs + k * VBN + tx * 4);
            const float4 b1 = *reinterpret_cast<const float4 *>(Bs + k * VBN + 64 + tx * 4);
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (more) vstore_slice(smem + ((t + 1) & 1) * VSTAGE, tid, ra, rb);
        __syncthreads();
    }

    const float alpha = g.alpha, beta = g.beta;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i >> 2) * 64 + ty * 4 + (i & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + (j >> 2) * 64 + tx * 4 + (j & 3);
            if (edge_mn && (row >= g.M || col >= g.N)) continue;
            float *p = g.C + (int64_t)row * g.ldc + col;
            float v = alpha * acc[i][j];
            if (beta != 0.f) v = fmaf(beta, *p, v);
            *p = v;
        }
    }
}

}  // namespace

int64_t valu_grid(int M, int N) {
    return (int64_t)((M + VBM - 1) / VBM) * ((N + VBN - 1) / VBN);
}

hipError_t launch_valu(const GemmArgs &g, bool vec_loads, hipStream_t stream) {
    const int tiles_m = (g.M + VBM - 1) / VBM;
    const int tiles_n = (g.N + VBN - 1) / VBN;
    const dim3 grid(tiles_m * tiles_n), block(VNT);
    if (vec_loads) hipLaunchKernelGGL((sgemm_valu_kernel<true>), grid, block, 0, stream, g, tiles_m, tiles_n, 8);
    else hipLaunchKernelGGL((sgemm_valu_kernel<false>), grid, block, 0, stream, g, tiles_m, tiles_n, 8);
    return hipGetLastError();
}

}  // namespace sgemm
