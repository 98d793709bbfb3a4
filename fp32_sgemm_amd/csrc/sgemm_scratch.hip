// Scratch memory of one call (split partial sums of the M <= 16 kernel and of
// split-K plans, the stream-K plan's partial tiles, the 16-bit GEMM's packed
// operands).
//
// The default entry points take it in stream order: hipMallocFromPoolAsync on
// the call's stream before its kernels, hipFreeAsync on the same stream after
// them, from a memory pool the library creates once per device.  The block is
// therefore valid exactly for the call's own kernels, calls on other streams
// never share it, nothing outlives the call, and both operations can be
// recorded into a graph.  The pool keeps up to kKeepBytes of freed memory for
// the next call instead of returning it to the driver at every
// synchronisation.  Every kernel writes the part of the scratch it later
// reads, so the memory is not cleared.
//
// A caller-provided region (Scratch::fixed, the allocation-free entry point)
// replaces the pool: acquire hands it out when it is large enough, release does
// nothing.
#include <cstdint>
#include <mutex>

#include "gemm_internal.hpp"

namespace sgemm {
namespace {

constexpr int kMaxDevices = 64;
constexpr uint64_t kKeepBytes = (uint64_t)1 << 30;

std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices] = {};

hipError_t device_pool(hipMemPool_t *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (g_pools[dev] == nullptr) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = kKeepBytes;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            hipMemPoolDestroy(pool);
            return e;
        }
        g_pools[dev] = pool;
    }
    *out = g_pools[dev];
    return hipSuccess;
}

}  // namespace

hipError_t scratch_acquire(const Scratch &s, size_t bytes, hipStream_t stream, void **out) {
    *out = nullptr;
    if (s.fixed != nullptr) {
        if (bytes > s.fixed_bytes) return hipErrorOutOfMemory;
        *out = s.fixed;
        return hipSuccess;
    }
    hipMemPool_t pool = nullptr;
    hipError_t e = device_pool(&pool);
    if (e != hipSuccess) return e;
    return hipMallocFromPoolAsync(out, bytes, pool, stream);
}

hipError_t scratch_release(const Scratch &s, void *p, hipStream_t stream) {
    if (s.fixed != nullptr || p == nullptr) return hipSuccess;
    return hipFreeAsync(p, stream);
}

}  // namespace sgemm
