// C = beta * C for the calls whose product term vanishes (alpha == 0 or
// K == 0).  With beta == 0 the kernel writes zeros and never reads C, so NaN
// or uninitialised memory in C does not propagate.
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

}  // namespace

hipError_t launch_scale_c(const GemmArgs &g, hipStream_t stream) {
    if (g.beta == 1.f) return hipSuccess;   // C unchanged
    const int64_t total = (int64_t)g.M * g.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(scale_c_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g.C, g.ldc, g.M, g.N, g.beta);
    return hipGetLastError();
}

}  // namespace sgemm
