// Workspace for kernels that need one (split partial sums of the M <= 16
// kernel, of split-K and stream-K plans, and the packed operands of the
// 16-bit-input GEMM).  The library keeps one workspace per (device, stream):
// work on one stream runs in order, so successive calls on a stream can reuse
// the same memory without further synchronisation, while calls on different
// streams never share it.  A stream's workspace is allocated on its first use
// and replaced by a block at least twice as large when a call needs more.  The
// old block is kept, not freed: work already queued on the stream, or a call
// from another host thread that obtained it a moment earlier, may still use
// it, and keeping it needs no synchronisation (the kept blocks together stay
// smaller than the current one).  Everything is held until the process ends.
// Every kernel writes the part of the workspace it later reads, so the memory
// is not cleared.
#include <cstdint>
#include <mutex>
#include <vector>

#include "gemm_internal.hpp"

namespace sgemm {
namespace {

struct Entry {
    int device;
    hipStream_t stream;
    void *ptr;
    size_t bytes;
};

std::mutex g_mutex;
std::vector<Entry> g_entries;
std::vector<void *> g_retired;   // replaced blocks, kept until the process ends

constexpr size_t kMinBytes = (size_t)4 << 20;

}  // namespace

hipError_t stream_workspace(size_t bytes, hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mutex);
    Entry *slot = nullptr;
    for (Entry &x : g_entries)
        if (x.device == dev && x.stream == stream) slot = &x;
    if (slot != nullptr && slot->bytes >= bytes) {
        *out = slot->ptr;
        return hipSuccess;
    }
    size_t want = bytes < kMinBytes ? kMinBytes : bytes;
    if (slot != nullptr && want < 2 * slot->bytes) want = 2 * slot->bytes;
    void *p = nullptr;
    e = hipMalloc(&p, want);
    if (e != hipSuccess) return e;
    if (slot == nullptr) {
        g_entries.push_back(Entry{dev, stream, p, want});
    } else {
        g_retired.push_back(slot->ptr);
        slot->ptr = p;
        slot->bytes = want;
    }
    *out = p;
    return hipSuccess;
}

}  // namespace sgemm
