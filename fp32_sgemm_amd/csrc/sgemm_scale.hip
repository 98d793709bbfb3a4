// C = beta * C for the calls whose product term vanishes (alpha == 0 or
// K == 0).  With beta == 0 the kernel writes zeros and never reads C, so NaN
// or uninitialised memory in C does not propagate.  Also the copy of an
// operand into rows that 16-byte loads can read.
#include "gemm_internal.hpp"

namespace sgemm {
namespace {

__global__ __launch_bounds__(256) void scale_c_kernel(float *C, int64_t ldc, int M, int N, float beta) {
    const int64_t total = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
        const int64_t i = t / N, j = t - i * N;
        float *p = C + i * ldc + j;
        *p = (beta == 0.f) ? 0.f : beta * *p;
    }
}

// Copies a rows x cols row-major matrix with row stride ld (any alignment)
// into rows of ld2 floats at dst (16-byte aligned, ld2 a multiple of 4),
// zeros past column cols.  Consecutive threads take consecutive groups of 4.
__global__ __launch_bounds__(256) void pack_rows_kernel(const float *src, int64_t ld, int rows, int cols, float *dst,
                                                        int64_t ld2) {
    const int64_t groups = ld2 / 4;
    const int64_t total = (int64_t)rows * groups;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
        const int64_t r = t / groups;
        const int c0 = (int)(t - r * groups) * 4;
        const float *s = src + r * ld;
        float4 v;
        v.x = c0 + 0 < cols ? s[c0 + 0] : 0.f;
        v.y = c0 + 1 < cols ? s[c0 + 1] : 0.f;
        v.z = c0 + 2 < cols ? s[c0 + 2] : 0.f;
        v.w = c0 + 3 < cols ? s[c0 + 3] : 0.f;
        *reinterpret_cast<float4 *>(dst + r * ld2 + c0) = v;
    }
}

}  // namespace

hipError_t launch_pack_rows(const float *src, int64_t ld, int rows, int cols, float *dst, int64_t ld2,
                            hipStream_t stream) {
    const int64_t total = (int64_t)rows * (ld2 / 4);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, ld, rows, cols, dst, ld2);
    return hipGetLastError();
}

hipError_t launch_scale_c(const GemmArgs &g, hipStream_t stream) {
    if (g.beta == 1.f) return hipSuccess;   // C unchanged
    const int64_t total = (int64_t)g.M * g.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(scale_c_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g.C, g.ldc, g.M, g.N, g.beta);
    return hipGetLastError();
}

}  // namespace sgemm
