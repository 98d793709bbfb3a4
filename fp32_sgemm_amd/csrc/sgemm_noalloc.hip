// The allocation-free entry point: sgemm_f32 whose scratch (the split partial
// sums of the M <= 32 kernel and of tuned split-K plans) is a fixed array in
// the library's device memory instead of a stream-ordered allocation.
//
// `scratch` below is a device variable: in host code its name is only a
// stand-in for the symbol, never a device address.  Its address on a device is
// looked up once per device (hipGetSymbolAddress with that device current, on
// the first call there) and only that address is passed on to the kernels.
#include <mutex>

#include "gemm_internal.hpp"
#include "sgemm_f32.h"

static constexpr size_t kScratchBytes = SGEMM_F32_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int sgemm_f32_noalloc(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                                 int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    sgemm::Scratch s;
    const hipError_t e = scratch_address(&s.fixed);
    if (e != hipSuccess) return -static_cast<int>(e);
    s.fixed_bytes = kScratchBytes;
    return sgemm::run_auto_with_scratch(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, s);
}
