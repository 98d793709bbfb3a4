// Internal declarations shared by the kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgemm {

// Where one call's scratch memory comes from: a caller-provided region
// (`fixed`, `fixed_bytes` long: the allocation-free entry point), or, when
// `fixed` is null, a stream-ordered allocation from the library's per-device
// memory pool.
struct Scratch {
    void *fixed = nullptr;
    size_t fixed_bytes = 0;
};

// Arguments of one C = alpha*op(A)*op(B) + beta*C call, row-major, strides in
// elements.  trans_a == 0: A is stored M x K; otherwise K x M and op(A) is its
// transpose.  trans_b == 0: B is stored K x N; otherwise N x K.  Only the MFMA
// kernels take transposed operands.
struct GemmArgs {
    int M, N, K;
    float alpha, beta;
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int trans_a = 0, trans_b = 0;
    Scratch scratch;
};

// Launchers: each enqueues its kernel(s) on `stream` and returns the HIP error
// of the launch.  Callers have validated the arguments, excluded M == 0,
// N == 0, and routed alpha == 0 / K == 0 to launch_scale_c.
hipError_t launch_mfma_large(const GemmArgs &g, bool vec_loads, hipStream_t stream);
// Copies rows x cols floats (row stride ld) into rows of ld2 floats at dst
// (16-byte aligned, ld2 a multiple of 4 and at least cols).
hipError_t launch_pack_rows(const float *src, int64_t ld, int rows, int cols, float *dst, int64_t ld2,
                            hipStream_t stream);
hipError_t launch_mfma_small(const GemmArgs &g, bool vec_loads, hipStream_t stream);

// MFMA tile configurations: 0 = 128x128 (the large tile), 1 = 64x64 (the
// small tile), 2 = 128x64, 3 = 64x128, 4 = 64x64 with two slices in flight,
// 5 = 128x128 persistent with stream-K (resident work-groups take whole tiles
// in rounds, then equal shares of the remaining tiles' K slices; split tiles
// are summed by a fix-up kernel), 6 = 64x64 with slices of 64, 7 = 256x256
// (sgemm_big.hip: one work-group per CU, operands copied straight into LDS),
// 8 = 128x128, 9 = 64x64 and 10 = 192x192 by the same kernel (two, four and
// one work-groups per CU).  Configurations 2-10 exist with 16-byte loads only.
// `group_m` is the number of tile rows walked together by the tile order
// (configuration 7 uses 4); `splits` divides K over work-groups (the partial
// sums go through the call's scratch and a reduction kernel; not with
// configurations 5 and 7-10).
constexpr int kNumMfmaConfigs = 11;
hipError_t launch_mfma_config(const GemmArgs &g, int config, bool vec_loads, int group_m, int splits,
                              hipStream_t stream);
int64_t mfma_config_tiles(int config, int M, int N);
bool mfma_config_scalar_ok(int config);
bool mfma_config_splits_ok(int config);
// Number of non-empty splits of K actually used for a requested count, and the
// K extent of each (a multiple of the tile depth).
int mfma_effective_splits(int K, int splits, int *k_per);
// 256 x 256 tiles, one work-group per CU (sgemm_big.hip): whether the
// product fits them (M, N, K multiples of 4, aligned operands), their count,
// and the launchers of the 256 x 256, 192 x 192, 128 x 128 and 64 x 64 grids.
bool big_tile_fits(const GemmArgs &g);   // operands (C's stride: big_tile_c_fits)
bool big_tile_c_fits(int64_t ldc);
int64_t big_tiles(int M, int N);
hipError_t launch_big(const GemmArgs &g, hipStream_t stream);
hipError_t launch_dl192(const GemmArgs &g, int group_m, hipStream_t stream);
hipError_t launch_dl128(const GemmArgs &g, int group_m, hipStream_t stream);
hipError_t launch_dl64(const GemmArgs &g, int group_m, hipStream_t stream);
hipError_t launch_valu(const GemmArgs &g, bool vec_loads, hipStream_t stream);
hipError_t launch_skinny(const GemmArgs &g, bool vec_loads, hipStream_t stream);
hipError_t launch_scale_c(const GemmArgs &g, hipStream_t stream);

// 16-bit-input GEMM (gemm16.hip).  The GemmArgs pointers A and B carry the
// 16-bit operands; kind is GEMM16_F32_BF16 or GEMM16_F32_F16.
hipError_t launch_gemm16(int kind, const GemmArgs &g, hipStream_t stream);
int64_t gemm16_grid(int M, int N);
// Tile size (256, 192 or 128) of the direct-to-LDS kernel for an M x N grid.
int gemm16_ring_tile(int M, int N);

// Scratch of at least `bytes` for the kernels a launcher is about to enqueue on
// `stream` (sgemm_scratch.hip), and its release after them (stream-ordered; a
// fixed region is handed out as it is and never released).  A launcher
// acquires before it enqueues anything, so a failed acquire leaves C alone.
// With a fixed region, a request larger than it fails with
// hipErrorOutOfMemory.
hipError_t scratch_acquire(const Scratch &s, size_t bytes, hipStream_t stream, void **out);
hipError_t scratch_release(const Scratch &s, void *p, hipStream_t stream);

// Scratch bytes that a launch will acquire (host side, no HIP call except the
// occupancy query of the stream-K plan): the M <= 32 kernel, an MFMA plan, and
// the 16-bit GEMM.
int64_t skinny_scratch_bytes(const GemmArgs &g);
hipError_t mfma_config_scratch_bytes(const GemmArgs &g, int config, int splits, int64_t *bytes);

// sgemm_f32's automatic GEMM with the call's scratch taken from `scratch`
// (sgemm_api.hip): validation, special cases and plan as sgemm_f32; with a
// fixed region, a plan that needs more scratch than it holds returns
// SGEMM_F32_ERR_SCRATCH before anything is enqueued.
int run_auto_with_scratch(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                          float beta, float *C, int ldc, hipStream_t stream, const Scratch &scratch);

// LDS poisoning, for a debug copy of the library only (compiled with
// -DSGEMM_LDS_POISON=1; the product is built without it): a kernel calls
// poison_lds on its LDS array first thing, which fills it with quiet NaNs and
// waits for every wave.  A stage that is read before the loads that fill it
// have landed, or a part of LDS that is read but never written, then turns
// the result into NaN instead of silently reading stale data or the zeros of a
// fresh work-group.
#ifndef SGEMM_LDS_POISON
#define SGEMM_LDS_POISON 0
#endif
template <int BYTES>
__device__ __forceinline__ void poison_lds(void *lds) {
    if constexpr (SGEMM_LDS_POISON != 0) {
        static_assert(BYTES % 4 == 0, "LDS size");
        float *p = static_cast<float *>(lds);
        for (int i = threadIdx.x; i < BYTES / 4; i += blockDim.x) p[i] = __builtin_nanf("");
        __syncthreads();
    }
}

// Tile counts that each launcher's grid uses (host side, for the size check).
int64_t mfma_large_grid(int M, int N);
int64_t mfma_small_grid(int M, int N);
int64_t valu_grid(int M, int N);
int64_t skinny_grid(const GemmArgs &g);

// The streaming kernels for a few rows of one side: which form serves a
// product (the plain form with rows of B streamed for M <= kSkinnyMaxM, B
// given N x K streamed along k for M <= 16, or A streamed along k for N <= 16
// with C written transposed), or -1 when none does or their 32-bit offsets do
// not cover the strides.
constexpr int kSkinnyMaxM = 32;
constexpr int kSkinnyRowsOfB = 0;
constexpr int kSkinnyBKMajor = 1;
constexpr int kSkinnyAKMajor = 2;
int skinny_form(int ta, int tb, int M, int N, int K, int64_t lda, int64_t ldb);

// ---------------------------------------------------------------------------
// Work-group to output-tile mapping.
//
// The hardware hands consecutive work-group ids to the 8 XCDs in turn
// (id % 8 picks the XCD), and each XCD has its own L2.  The mapping first
// renumbers ids so that each XCD receives one contiguous run of tile numbers,
// then walks tile numbers in groups of `group_m` tile rows, column by column
// inside a group, so that the work-groups resident on one XCD at the same time
// cover a compact block of C and share the A row-panels and B column-panels
// they stream through that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

// Tile t of the grouped order: groups of `group_m` tile rows, column by column
// inside a group.
__host__ __device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int &tm,
                                                     int &tn) {
    const int in_group = group_m * tiles_n;
    const int g = t / in_group;
    const int first_m = g * group_m;
    const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int r = t - g * in_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// Work-group id -> position in an XCD-contiguous order: XCD x (= id % 8)
// receives positions [x*per + min(x, rem), ...) in launch order.
__host__ __device__ __forceinline__ int xcd_position(int bid, int total) {
    const int per = total / kNumXcd;
    const int rem = total % kNumXcd;
    const int xcd = bid % kNumXcd;
    const int local = bid / kNumXcd;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__host__ __device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n,
                                              int group_m, int &tm, int &tn) {
    tile_coords(xcd_position(bid, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace sgemm
