// Scratch memory of one call (split partial sums of the M <= 32 kernel and of
// split-K plans, the stream-K plan's partial tiles, the 16-bit GEMM's packed
// operands).
//
// Eager calls (the stream is not being captured) reuse a block cached for
// their device and stream handle.  Calls on one stream run in order, so the
// block needs no synchronisation; a block never passes to another stream.  (A
// handle can name a new stream only after the old one was destroyed, which
// waits for the old stream's work.)  A block
// too small for a call is freed in the order of its own stream and a larger one
// taken.  At most kMaxCached streams get a block (they keep it until the
// process ends), each at most kCacheMaxBytes; other streams and larger
// requests take pool memory per call as below.  (A stream-ordered allocation
// and free around every call cost about 17 us of host time per call, more
// than the kernels of a 16 x 4096 x 4096 product take on the GPU, and an event
// recorded after every call to hand blocks between streams cost 2.7 us of GPU
// time per call.)
//
// Calls recorded into a graph (the stream is capturing), and the cases above,
// take their scratch in stream order: hipMallocFromPoolAsync on the call's
// stream before its kernels, hipFreeAsync after them, from a memory pool the
// library creates once per device; under capture both become nodes of the
// graph.  The pool keeps up to kKeepBytes of freed memory for the next call.
// Cached blocks come from the same pool.  Every kernel writes the part of the
// scratch it later reads, so the memory is not cleared.
//
// A caller-provided region (Scratch::fixed, the allocation-free entry point)
// replaces both: acquire hands it out when it is large enough, release does
// nothing.
#include <cstdint>
#include <mutex>

#include "gemm_internal.hpp"

namespace sgemm {
namespace {

constexpr int kMaxDevices = 64;
constexpr uint64_t kKeepBytes = (uint64_t)1 << 30;
constexpr int kMaxCached = 8;                       // cached blocks (device, stream)
constexpr size_t kCacheMaxBytes = (size_t)64 << 20; // largest cached block
constexpr size_t kGranule = (size_t)1 << 20;        // cached blocks grow in whole MiB

std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices] = {};

hipError_t device_pool(int dev, hipMemPool_t *out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (g_pools[dev] == nullptr) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        hipError_t e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = kKeepBytes;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return e;
        }
        g_pools[dev] = pool;
    }
    *out = g_pools[dev];
    return hipSuccess;
}

struct Cached {
    int dev = -1;
    hipStream_t stream = nullptr;
    void *ptr = nullptr;
    size_t bytes = 0;
    int holders = 0;             // calls between acquire and release
};

std::mutex g_cache_mutex;
Cached g_cache[kMaxCached];

hipError_t pool_acquire(int dev, size_t bytes, hipStream_t stream, void **out) {
    hipMemPool_t pool = nullptr;
    hipError_t e = device_pool(dev, &pool);
    if (e != hipSuccess) return e;
    return hipMallocFromPoolAsync(out, bytes, pool, stream);
}

// The cached block of (dev, stream), made or grown to at least `bytes`; sets
// *out to nullptr when there is none to use (every slot taken by other
// streams, or the block must grow while another call on the stream holds it).
hipError_t cached_acquire(int dev, size_t bytes, hipStream_t stream, void **out) {
    *out = nullptr;
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    Cached *c = nullptr;
    for (Cached &x : g_cache)
        if (x.ptr != nullptr && x.dev == dev && x.stream == stream) c = &x;
    if (c == nullptr) {
        for (Cached &x : g_cache)
            if (x.ptr == nullptr && c == nullptr) c = &x;
        if (c == nullptr) return hipSuccess;
        c->dev = dev;
        c->stream = stream;
        c->holders = 0;
    } else if (c->bytes < bytes) {
        if (c->holders > 0) return hipSuccess;
        // In stream order, after the calls that used it.
        const hipError_t e = hipFreeAsync(c->ptr, stream);
        c->ptr = nullptr;
        c->bytes = 0;
        if (e != hipSuccess) return e;
    }
    if (c->ptr == nullptr) {
        const size_t want = (bytes + kGranule - 1) / kGranule * kGranule;
        const hipError_t e = pool_acquire(dev, want, stream, &c->ptr);
        if (e != hipSuccess) {
            c->ptr = nullptr;
            return e;
        }
        c->bytes = want;
    }
    ++c->holders;
    *out = c->ptr;
    return hipSuccess;
}

// After the call's kernels.  False when `p` is not a cached block (pool memory).
bool cached_release(void *p) {
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    for (Cached &x : g_cache) {
        if (x.ptr == p && x.holders > 0) {
            --x.holders;
            return true;
        }
    }
    return false;
}

}  // namespace

hipError_t scratch_acquire(const Scratch &s, size_t bytes, hipStream_t stream, void **out) {
    *out = nullptr;
    if (s.fixed != nullptr) {
        if (bytes > s.fixed_bytes) return hipErrorOutOfMemory;
        *out = s.fixed;
        return hipSuccess;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap == hipStreamCaptureStatusNone && bytes <= kCacheMaxBytes) {
        e = cached_acquire(dev, bytes, stream, out);
        if (e != hipSuccess || *out != nullptr) return e;
    }
    return pool_acquire(dev, bytes, stream, out);
}

hipError_t scratch_release(const Scratch &s, void *p, hipStream_t stream) {
    if (s.fixed != nullptr || p == nullptr) return hipSuccess;
    if (cached_release(p)) return hipSuccess;
    return hipFreeAsync(p, stream);
}

}  // namespace sgemm
