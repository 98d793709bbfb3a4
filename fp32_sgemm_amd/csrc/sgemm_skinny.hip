// FP32 GEMM for M <= 32 (a short, wide A times a tall B), on 16x16x4 MFMA.
//
// With M = 16 and N = K = 4096 the product does 8 FLOP per byte of B it must
// stream, below the MI355X ridge point of about 20 FLOP per byte, so the kernel
// is bound by HBM bandwidth: its job is to stream B exactly once, in row
// segments long enough for the memory system (256 bytes) and with enough loads
// in flight.  (Decode-time GEMV-like shapes sit on the bandwidth roof, "Writing
// a Fast Matmul in CUDA, Step by Step", section "In the real world"; too few
// output tiles to fill the machine is where the reduction is split, "How a
// Matmul Kernel Gets Fast", section 15.)
//
// Work decomposition.  A work-group owns a 64-column strip of C and one of
// `splits` contiguous ranges of K; its 4 waves split that range again, each
// streaming its part in batches of 16 rows, two batches in flight.  The
// partial strips of the splits go to the call's scratch and a second kernel
// adds them in split order and finishes C (with one split, the first kernel
// finishes C itself).  B is read once, so its loads are marked non-temporal:
// through the library, 16 x 4096 x 4096 with B over 7 copies (past the
// Infinity Cache), calls back to back between one pair of events, 20.6-20.9
// us per call with plain loads and batches of 32 rows, 19.2-19.7 with
// non-temporal loads, 17.7-18.6 with batches of 16 rows as well (8 x 4096 x
// 4096: 20.1 -> 17.5-17.6; 16 x 11008 x 4096: 49.0 -> 46.4; bit for bit the
// same sums on the 4096-wide shapes); batches of 48 or 64 rows were slower
// (19.3, 24.9), and so were four work-groups per CU (21.4) or one (21.3),
// except at N = 11008 (42.9 with four), and 2 or 8 waves per work-group
// (23.6, 19.1).  Measured alternatives before those
// changes, the same workload:
//   - this form, 8 splits: 18.9-19.0 us per call, its first kernel alone
//     16.8 us; a kernel that only reads B with the same decomposition takes
//     14.7 us and the fastest plain read of B found 12.6 us (12.3 with
//     non-temporal loads);
//   - the same kernels fused, the last split of each strip adding the others'
//     partials once their flags show the call's epoch (agent-scope coherent
//     stores and loads, no fences): 19.3-19.4 us, the waiting tail costs more
//     than the second launch;
//   - A staged in LDS per work-group instead of read with B: 21.9 us (fused);
//   - 4 batches per wave, or batches interleaved across the waves: 21-22 us;
//     16 splits: 24.1 us.
// With events around every call (each pair costs GPU time here):
//   - no split between work-groups (a work-group per strip of 16, 32 or 64
//     columns with 4-16 waves splitting K, reduced in LDS, no scratch at all):
//     30-40 us, too few bytes of B in flight per strip;
//   - wider strips (256 or 512 columns per work-group) or more waves: 26-37 us;
//   - the last work-group of a strip to finish adding the partials (a
//     device-scope counter): no gain with coherent partial stores and loads,
//     38.8 us with release/acquire fences (each fence writes back or
//     invalidates a whole L2).
//
// M = 17..32 takes two blocks of 16 rows of A (twice the MFMAs per byte of B;
// at 32 rows the fp32 MFMA work per SIMD is about 80 % of the time the SIMD's
// share of HBM bandwidth takes to stream the batches, so loads must stay in
// flight under the MFMAs).  Grids of at most 64 strips keep three batches in
// flight per wave, wider grids two.  Per call, B over 7 copies, against the
// plan such shapes took before (64 x 64 MFMA tiles, K split 4 or 8 ways): 17 x 4096 x 4096
// 24.2 -> 20.1 us, 32 x 4096 x 4096 24.1 -> 21.5, 32 x 2048 x 8192 27.4 ->
// 22.1, 32 x 4096 x 11008 51.5 -> 45.4, 20 x 11008 x 4096 54.4 -> 55.6; two
// batches in flight everywhere: 21.6, 23.0, 23.5, 46.1, 54.5; three
// everywhere with two work-groups per CU (182 registers per lane): 20 x 11008
// x 4096 at 66.2 (516 work-groups, 4 past one round).  M <= 16 with three in
// flight: 8 x 4096 x 4096 18.1 -> 17.2 us, 16 x 4096 x 4096 17.9 -> 17.6.
//
// Inner step.  For a block of 16 rows of B starting at kb, lane l (h = l/16,
// j = l%16) loads columns 4j..4j+3 of rows kb + 4h + q, q = 0..3 (four 16-byte
// loads: 4 rows x 256 bytes per wave instruction), and A(j, kb + 4h .. +3) (one
// 16-byte load).  Element e of the B group is the operand of the e-th of four
// v_mfma_f32_16x16x4_f32 that accumulate columns 4j + e of the strip, so no
// data is reshuffled: the MFMA's column index j stands for strip column 4j + e.
// In the q-th step lane l supplies k = kb + 4h + q, with A from component q of
// its A group.
//
// All loads are buffer loads against resources that end at the last valid
// element of the batch: rows of A past M and rows of B past the split's range
// read as zeros by themselves; groups past column N of B or past the range's
// last k of A get an out-of-range lane offset, and groups that straddle those
// edges are loaded element by element.  Nothing outside the matrices is read.
#include "gemm_internal.hpp"

namespace sgemm {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ f32x4v sk_buffer_load_v4f32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.v4f32");
__device__ float sk_buffer_load_f32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.f32");

constexpr int kOff = (int)0x80000000u;   // past every extent used here: reads zero, no access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes, 0x00020000);
}

constexpr int SK_NW = 4;                 // waves per work-group
constexpr int SK_NT = SK_NW * 64;
constexpr int SK_BN = 64;                // columns of C per work-group
constexpr int SK_U = 1;                  // 16-row blocks per batch
constexpr int SK_ROWS = SK_U * 16;       // rows of B per batch

struct SkinnyArgs {
    GemmArgs g;
    float *ws;            // splits x M x N partial sums (unused with one split)
    int splits;
    int split_rows;       // rows of K per split, a multiple of SK_ROWS
};

// Four consecutive elements of one row at byte offset `off` of resource `r`,
// starting `col` elements into the row; elements at or past `limit` read as
// zero.  VEC: one 16-byte load when the group lies inside.  AUX: the loads'
// cache-policy bits.
template <bool VEC, int AUX>
__device__ __forceinline__ float4 load_group(__amdgpu_buffer_rsrc_t r, int off, int col, int limit) {
    float4 v;
    if (VEC && col + 3 < limit) {
        const f32x4v w = sk_buffer_load_v4f32(r, off, 0, AUX);
        v = make_float4(w[0], w[1], w[2], w[3]);
    } else if (VEC && col >= limit) {
        v = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        v.x = sk_buffer_load_f32(r, col + 0 < limit ? off + 0 : kOff, 0, AUX);
        v.y = sk_buffer_load_f32(r, col + 1 < limit ? off + 4 : kOff, 0, AUX);
        v.z = sk_buffer_load_f32(r, col + 2 < limit ? off + 8 : kOff, 0, AUX);
        v.w = sk_buffer_load_f32(r, col + 3 < limit ? off + 12 : kOff, 0, AUX);
    }
    return v;
}

// B is read once: its loads are marked non-temporal.
constexpr int kStreamAux = 2;

// Grids of at most this many strips keep three batches in flight per wave,
// wider ones two (their splits are longer and the third batch's registers
// cost more than it hides).
constexpr int kDeepStrips = 64;

// MB blocks of 16 rows of A (M <= 16 MB); row m of A is lane m % 16's in block m / 16.
template <int MB>
struct Batch {
    float4 a[SK_U][MB];
    float4 b[SK_U][4];
};

// Loads the batch whose first row of B (column of A) is kb; rows at or past
// kend belong to another split or lie past K and read as zero.
template <bool VEC, int MB>
__device__ __forceinline__ void load_batch(const GemmArgs &g, int n0, int kb, int kend, int lane, Batch<MB> &bt) {
    const int rows = min(SK_ROWS, kend - kb);
    const int cols = min(SK_BN, g.N - n0);
    const __amdgpu_buffer_rsrc_t rb = sk_rsrc(g.B + (int64_t)kb * g.ldb + n0,
                                              (int)(((int64_t)(rows - 1) * g.ldb + cols) * 4));
    const __amdgpu_buffer_rsrc_t ra = sk_rsrc(g.A + kb, (int)(((int64_t)(g.M - 1) * g.lda + rows) * 4));
    const int h = lane >> 4, j = lane & 15;
#pragma unroll
    for (int u = 0; u < SK_U; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = u * 16 + 4 * h + q;                  // row of B within the batch
            bt.b[u][q] = load_group<VEC, kStreamAux>(rb, (int)((r * g.ldb + 4 * j) * 4), 4 * j, r < rows ? cols : 0);
        }
        const int k = u * 16 + 4 * h;                          // first k of this lane's A groups
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = 16 * mb + j;
            bt.a[u][mb] = load_group<VEC, 0>(ra, (int)((m * g.lda + k) * 4), k, m < g.M ? rows : 0);
        }
    }
}

template <int MB>
__device__ __forceinline__ void consume_batch(const Batch<MB> &bt, f32x4v (&acc)[MB][4]) {
#pragma unroll
    for (int u = 0; u < SK_U; ++u) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const float av[4] = {bt.a[u][mb].x, bt.a[u][mb].y, bt.a[u][mb].z, bt.a[u][mb].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 b = bt.b[u][q];
                acc[mb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], b.x, acc[mb][0], 0, 0, 0);
                acc[mb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], b.y, acc[mb][1], 0, 0, 0);
                acc[mb][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], b.z, acc[mb][2], 0, 0, 0);
                acc[mb][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], b.w, acc[mb][3], 0, 0, 0);
            }
        }
    }
}

// DEPTH batches in flight per wave (2 or 3).  Two blocks of A with three
// batches in flight would take 182 registers per lane and fit only two
// work-groups per compute unit: the launch bound asks for three.
template <bool VEC, int MB, int DEPTH>
__global__ __launch_bounds__(SK_NT, MB == 2 ? 3 : 1) void sgemm_skinny_kernel(SkinnyArgs sa, int strips) {
    __shared__ float red[SK_NW][16 * MB * SK_BN];
    poison_lds<sizeof(red)>(red);
    const GemmArgs &g = sa.g;
    // Work-group -> (split, strip); consecutive strips stay on one XCD.
    int split, strip;
    tile_of_block(blockIdx.x, sa.splits, strips, 1, split, strip);
    const int n0 = strip * SK_BN;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    const int kbeg = split * sa.split_rows;
    const int kend = min(g.K, kbeg + sa.split_rows);
    // Contiguous part of the split for this wave, in whole batches.
    const int batches = (kend - kbeg + SK_ROWS - 1) / SK_ROWS;
    const int per_wave = (batches + SK_NW - 1) / SK_NW;
    const int bbeg = wave * per_wave;
    const int bend = min(batches, bbeg + per_wave);

    f32x4v acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][e] = f32x4v{0.f, 0.f, 0.f, 0.f};
    int b = bbeg;
    // The loads in the loops are unconditional (past the end they re-read the
    // wave's last batch, which is then not consumed) so the wait counts stay
    // exact.
    auto kof = [&](int bi) { return kbeg + (bi < bend ? bi : bend - 1) * SK_ROWS; };
    if constexpr (DEPTH == 2) {
        Batch<MB> b0, b1;
        if (b < bend) load_batch<VEC>(g, n0, kof(b), kend, lane, b0);
        for (; b + 1 < bend; b += 2) {
            load_batch<VEC>(g, n0, kof(b + 1), kend, lane, b1);
            consume_batch(b0, acc);
            load_batch<VEC>(g, n0, kof(b + 2), kend, lane, b0);
            consume_batch(b1, acc);
        }
        if (b < bend) consume_batch(b0, acc);
    } else {
        // Three batches in flight: two loaded ahead of the one consumed.
        Batch<MB> b0, b1, b2;
        if (b < bend) {
            load_batch<VEC>(g, n0, kof(b), kend, lane, b0);
            load_batch<VEC>(g, n0, kof(b + 1), kend, lane, b1);
        }
        for (; b + 2 < bend; b += 3) {
            load_batch<VEC>(g, n0, kof(b + 2), kend, lane, b2);
            consume_batch(b0, acc);
            load_batch<VEC>(g, n0, kof(b + 3), kend, lane, b0);
            consume_batch(b1, acc);
            load_batch<VEC>(g, n0, kof(b + 4), kend, lane, b1);
            consume_batch(b2, acc);
        }
        if (b < bend) consume_batch(b0, acc);
        if (b + 1 < bend) consume_batch(b1, acc);
    }

    // acc[mb][e] register r of lane l holds row 16*mb + 4*(l/16) + r, strip
    // column 4*(l%16) + e.  Add the waves' partials in wave order.
    const int h = lane >> 4, j = lane & 15;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][(16 * mb + 4 * h + r) * SK_BN + 4 * j + e] = acc[mb][e][r];
    __syncthreads();
    constexpr int PER_T = 16 * MB * SK_BN / SK_NT;   // strip elements per thread
    float part[PER_T];
#pragma unroll
    for (int t = 0; t < PER_T; ++t) {
        const int idx = threadIdx.x + t * SK_NT;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < SK_NW; ++w) s += red[w][idx];
        part[t] = s;
    }

#pragma unroll
    for (int t = 0; t < PER_T; ++t) {
        const int idx = threadIdx.x + t * SK_NT;
        const int row = idx / SK_BN, col = idx % SK_BN;
        if (row < g.M && n0 + col < g.N) {
            if (sa.splits > 1) {
                sa.ws[((int64_t)split * g.M + row) * g.N + n0 + col] = part[t];
            } else {
                float *p = g.C + (int64_t)row * g.ldc + n0 + col;
                float v = g.alpha * part[t];
                if (g.beta != 0.f) v = fmaf(g.beta, *p, v);
                *p = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streamed operand with rows contiguous in k.  D(i, r) = sum_k X(i, k) W(r, k)
// for at most 16 rows i of a small operand X and many rows r of W:
//   - B given N x K (NT, TT) with M <= 16: X = op(A), W = B as stored, D = C;
//   - A as given with N <= 16 (NN, NT): X = op(B) transposed, W = A, D = C
//     transposed.
// A work-group owns 32 rows of W (two groups of 16) and one range of K, split
// again over its 4 waves in batches of 64 k.  In a batch, lane l (h = l/16,
// j = l%16) loads W(r0 + 16 g + j, kb + 16 q + 4 h .. +3) for g = 0, 1 and
// q = 0..3 (each load: 16 rows x 64 bytes, a row's 256 bytes over the four
// q) and X(j, the same k) likewise.  Component e of the q-th groups is the
// k = kb + 16 q + 4 h + e operand of one 16x16x4 MFMA per g: lane
// (j, h) supplies row j of X and column j of W at the h-th k, so the product
// needs no reshuffling.  X given transposed (k-major) is read element by
// element.  Partial sums go to scratch in C's order when K is split over
// work-groups, and the same ordered reduction finishes C.
constexpr int KM_RW = 32;                // rows of W per work-group
constexpr int KM_G = KM_RW / 16;         // groups of 16 rows of W
constexpr int KM_BK = 64;                // k per batch
constexpr int KM_RED = KM_RW + 1;        // padded row of the LDS reduction
constexpr int kKMajorMaxRows = 16;       // rows of X
// Three batches in flight per wave where each wave streams at least
// kDeepBatches batches of its split, two otherwise (per call, both operands
// cycled past the Infinity Cache, two -> three: NT 16 x 11008 x 4096 53.3 ->
// 50.4 us, NN 11008 x 16 x 4096 50.2 -> 46.9, with 8 batches per wave; NT
// 16 x 4096 x 4096 22.8 -> 23.7 with 4).
constexpr int kDeepBatches = 6;
// Splits of 512 to KM_XL_ROWS k with X read along k stage each wave's part
// of X in LDS (rows of KM_XS floats: the part's KM_XL_ROWS / 4 k and a pad
// that spreads the 16 rows over the banks): per call, both operands cycled,
// NT 16 x 4096 x 4096 22.9 -> 21.0 us, NT 16 x 2048 x 8192 23.2 -> 21.0, NT
// 4096 x 16 x 4096 23.0 -> 21.0.  Staging k-major X (16 scalar loads per k
// row pass, written across rows) lost: TT 16 x 4096 x 4096 21.2 -> 26.0, NN
// 4096 x 16 x 4096 21.3 -> 26.3; so did one batch per wave (NT 8 x 1024 x
// 1024 7.2 -> 8.8).
constexpr int KM_XL_ROWS = 1024;
constexpr int KM_XS = KM_XL_ROWS / SK_NW + 4;

struct KmajArgs {
    const float *W;
    int64_t ldw;
    int R;                // rows of W
    const float *X;
    int64_t x_si, x_sk;   // X(i, k) at X[i * x_si + k * x_sk]
    int MX;               // rows of X (<= 16)
    int K;
    float alpha, beta;
    float *C;
    int64_t c_si, c_sr;   // D(i, r) at C[i * c_si + r * c_sr]
    float *ws;            // splits x MX x R partial sums in C's order
    int64_t w_si, w_sr;
    int splits;
    int split_rows;       // k per split, a multiple of KM_BK
};

struct KBatch {
    float4 w[KM_G][4];
    float4 x[4];
};

template <bool VEC, bool XT, bool XL>
__device__ __forceinline__ void kmaj_load(const KmajArgs &a, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                          int rows, int kb, int kend, int h, int j, KBatch &bt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = kb + 16 * q + 4 * h;       // first k of this lane's groups
#pragma unroll
        for (int g = 0; g < KM_G; ++g) {
            const int r = 16 * g + j;            // row of W within the work-group's rows
            bt.w[g][q] = load_group<VEC, 0>(rw, (int)((r * a.ldw + k) * 4), k, r < rows ? kend : 0);
        }
        if (XL) {                                // X comes from the wave's LDS slice
        } else if (XT) {                         // X(j, k..k+3) lies down a column
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = sk_buffer_load_f32(rx, j < a.MX && k + e < kend ? (int)(((k + e) * a.x_sk + j) * 4) : kOff, 0, 0);
            bt.x[q] = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            bt.x[q] = load_group<VEC, 0>(rx, (int)((j * a.x_si + k) * 4), k, j < a.MX ? kend : 0);
        }
    }
}

__device__ __forceinline__ float comp(const float4 &v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

__device__ __forceinline__ void kmaj_consume(const KBatch &bt, f32x4v (&acc)[KM_G]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = comp(bt.x[q], e);
#pragma unroll
            for (int g = 0; g < KM_G; ++g)
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, comp(bt.w[g][q], e), acc[g], 0, 0, 0);
        }
}

// TOUT: D is C transposed (consecutive threads then write consecutive i).
// MODE 0: two batches in flight; 1: three; 2: two, with X (read along k)
// staged once per wave in LDS (splits of at most KM_XL_ROWS k: a wave's part
// is at most KM_XL_ROWS / 4 k).
template <bool VEC, bool XT, bool TOUT, int MODE>
__global__ __launch_bounds__(SK_NT, 2) void sgemm_kmaj_kernel(KmajArgs a, int strips) {
    constexpr bool XL = MODE == 2;
    constexpr int DEPTH = MODE == 1 ? 3 : 2;
    // Per wave: its X slice (16 rows of KM_XS floats) when staged, then the
    // partial strip for the reduction (which overwrites the slice).
    constexpr int WSTRIDE = XL ? 16 * KM_XS : 16 * KM_RED;
    __shared__ __align__(16) float lds[SK_NW * WSTRIDE];
    poison_lds<sizeof(lds)>(lds);
    int split, strip;
    tile_of_block(blockIdx.x, a.splits, strips, 1, split, strip);
    const int r0 = strip * KM_RW;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int h = lane >> 4, j = lane & 15;

    const int kbeg = split * a.split_rows;
    const int kend = min(a.K, kbeg + a.split_rows);
    const int batches = (kend - kbeg + KM_BK - 1) / KM_BK;
    const int per_wave = (batches + SK_NW - 1) / SK_NW;
    const int bbeg = wave * per_wave;
    const int bend = min(batches, bbeg + per_wave);

    // Resources over this work-group's rows of W and over all of X: rows
    // past R and k past the range read as zero.
    const int rows = min(KM_RW, a.R - r0);
    const __amdgpu_buffer_rsrc_t rw = sk_rsrc(a.W + (int64_t)r0 * a.ldw, (int)(((rows - 1) * a.ldw + a.K) * 4));
    const __amdgpu_buffer_rsrc_t rx =
        sk_rsrc(a.X, XT ? (int)(((a.K - 1) * a.x_sk + a.MX) * 4) : (int)(((a.MX - 1) * a.x_si + a.K) * 4));

    f32x4v acc[KM_G];
#pragma unroll
    for (int g = 0; g < KM_G; ++g) acc[g] = f32x4v{0.f, 0.f, 0.f, 0.f};
    int b = bbeg;
    // As in the other kernel: unconditional loads in the loops, past the end
    // re-reading the wave's last batch, which is then not consumed.
    auto kof = [&](int bi) { return kbeg + (bi < bend ? bi : bend - 1) * KM_BK; };
    float *xs = lds + wave * WSTRIDE;
    if constexpr (XL) {
        static_assert(!XT, "X is staged where it is read along k");
        // This wave's X(0..15, ks .. ks + KM_XL_ROWS / 4), zero past its
        // range and past MX, read with whole-row loads (64 lanes x 16 bytes of
        // one row of X) and written to LDS as rows of KM_XS floats.  Only
        // this wave reads it, so no barrier orders it.
        KBatch b0, b1;
        if (b < bend) {
            const int ks = kbeg + bbeg * KM_BK;
            const int ke = min(kend, kbeg + bend * KM_BK);
            float4 v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = load_group<VEC, 0>(rx, (int)((i * a.x_si + ks + 4 * lane) * 4), ks + 4 * lane,
                                          i < a.MX ? ke : 0);
            // The first batch of W goes out before the X rows are written.
            kmaj_load<VEC, XT, true>(a, rw, rx, rows, kof(b), kend, h, j, b0);
#pragma unroll
            for (int i = 0; i < 16; ++i) *reinterpret_cast<float4 *>(xs + i * KM_XS + 4 * lane) = v[i];
        }
        auto xfrag = [&](int bi, KBatch &bt) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bt.x[q] = *reinterpret_cast<const float4 *>(xs + j * KM_XS + (bi - bbeg) * KM_BK + 16 * q + 4 * h);
        };
        for (; b + 1 < bend; b += 2) {
            kmaj_load<VEC, XT, true>(a, rw, rx, rows, kof(b + 1), kend, h, j, b1);
            xfrag(b, b0);
            kmaj_consume(b0, acc);
            kmaj_load<VEC, XT, true>(a, rw, rx, rows, kof(b + 2), kend, h, j, b0);
            xfrag(b + 1, b1);
            kmaj_consume(b1, acc);
        }
        if (b < bend) {
            xfrag(b, b0);
            kmaj_consume(b0, acc);
        }
    } else if constexpr (DEPTH == 2) {
        KBatch b0, b1;
        if (b < bend) kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b), kend, h, j, b0);
        for (; b + 1 < bend; b += 2) {
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b + 1), kend, h, j, b1);
            kmaj_consume(b0, acc);
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b + 2), kend, h, j, b0);
            kmaj_consume(b1, acc);
        }
        if (b < bend) kmaj_consume(b0, acc);
    } else {
        KBatch b0, b1, b2;
        if (b < bend) {
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b), kend, h, j, b0);
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b + 1), kend, h, j, b1);
        }
        for (; b + 2 < bend; b += 3) {
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b + 2), kend, h, j, b2);
            kmaj_consume(b0, acc);
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b + 3), kend, h, j, b0);
            kmaj_consume(b1, acc);
            kmaj_load<VEC, XT, false>(a, rw, rx, rows, kof(b + 4), kend, h, j, b1);
            kmaj_consume(b2, acc);
        }
        if (b < bend) kmaj_consume(b0, acc);
        if (b + 1 < bend) kmaj_consume(b1, acc);
    }

    // acc[g] register r of lane (j, h) holds i = 4 h + r, row r0 + 16 g + j
    // of W.  The waves' partials are added in wave order.
#pragma unroll
    for (int g = 0; g < KM_G; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[(4 * h + r) * KM_RED + 16 * g + j] = acc[g][r];
    __syncthreads();
    constexpr int NI = 16;
    constexpr int PER_T = NI * KM_RW / SK_NT;
#pragma unroll
    for (int t = 0; t < PER_T; ++t) {
        const int idx = threadIdx.x + t * SK_NT;
        const int i = TOUT ? idx % NI : idx / KM_RW;
        const int c = TOUT ? idx / NI : idx % KM_RW;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < SK_NW; ++w) s += lds[w * WSTRIDE + i * KM_RED + c];
        if (i < a.MX && r0 + c < a.R) {
            const int64_t r = r0 + c;
            if (a.splits > 1) {
                a.ws[(int64_t)split * a.MX * a.R + i * a.w_si + r * a.w_sr] = s;
            } else {
                float *p = a.C + i * a.c_si + r * a.c_sr;
                float v = a.alpha * s;
                if (a.beta != 0.f) v = fmaf(a.beta, *p, v);
                *p = v;
            }
        }
    }
}

// C = alpha * (sum of the split partials, in split order) + beta * C.  The
// partials' loads go out eight at a time before their additions (with a
// run-time loop bound each addition would wait for its own load, one memory
// round trip per split); indices past the last split re-read it and are not
// added.
__global__ __launch_bounds__(256) void skinny_reduce_kernel(GemmArgs g, const float *ws, int splits) {
    const int64_t total = (int64_t)g.M * g.N;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int sp0 = 0; sp0 < splits; sp0 += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = ws[(sp0 + j < splits ? sp0 + j : splits - 1) * total + t];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (sp0 + j < splits) s += v[j];
        }
        const int64_t i = t / g.N, jj = t - i * g.N;
        float *p = g.C + i * g.ldc + jj;
        float v = g.alpha * s;
        if (g.beta != 0.f) v = fmaf(g.beta, *p, v);
        *p = v;
    }
}

}  // namespace

namespace {

constexpr int64_t kOffsetLimit = (int64_t)1 << 31;

bool rows_fit(int64_t lda, int64_t ldb) {
    // One batch of B and all kSkinnyMaxM rows of A must be addressable with
    // 32-bit byte offsets.
    return ((int64_t)SK_ROWS * ldb + SK_BN) * 4 < kOffsetLimit && ((int64_t)kSkinnyMaxM * lda + SK_ROWS) * 4 < kOffsetLimit;
}

// A work-group's rows of W, and all of X (MX rows, given k-major when xt),
// must be addressable with 32-bit byte offsets.
bool kmaj_fits(int64_t ldw, int64_t ldx, bool xt, int MX, int K) {
    const bool w_ok = ((int64_t)(KM_RW - 1) * ldw + K) * 4 < kOffsetLimit;
    const bool x_ok = xt ? ((int64_t)(K - 1) * ldx + MX) * 4 < kOffsetLimit
                         : ((int64_t)(MX - 1) * ldx + K) * 4 < kOffsetLimit;
    return w_ok && x_ok;
}

}  // namespace

int skinny_form(int ta, int tb, int M, int N, int K, int64_t lda, int64_t ldb) {
    if (!ta && !tb && M <= kSkinnyMaxM && rows_fit(lda, ldb)) return kSkinnyRowsOfB;
    if (tb && M <= kKMajorMaxRows && kmaj_fits(ldb, lda, ta != 0, M, K)) return kSkinnyBKMajor;
    if (!ta && N <= kKMajorMaxRows && kmaj_fits(lda, ldb, tb == 0, N, K)) return kSkinnyAKMajor;
    return -1;
}

int64_t skinny_grid(const GemmArgs &g) {
    const int form = skinny_form(g.trans_a, g.trans_b, g.M, g.N, g.K, g.lda, g.ldb);
    if (form == kSkinnyRowsOfB) return (g.N + SK_BN - 1) / SK_BN;
    return ((form == kSkinnyBKMajor ? g.N : g.M) + (int64_t)KM_RW - 1) / KM_RW;
}

namespace {

// Work-groups wanted per call: two per compute unit.
constexpr int kSkinnySlots = 512;

// The K split over `strips` work-group columns: about kSkinnySlots work-groups,
// every split at least 256 k long and a whole number of batches of `unit` k.
void skinny_split(int strips, int K, int unit, int *splits_out, int *split_rows_out) {
    const int want = (kSkinnySlots + strips - 1) / strips;
    const int max_splits = (K + 255) / 256;
    int splits = want < max_splits ? want : max_splits;
    if (splits < 1) splits = 1;
    int split_rows = (K + splits - 1) / splits;
    split_rows = (split_rows + unit - 1) / unit * unit;
    splits = (K + split_rows - 1) / split_rows;
    *splits_out = splits;
    *split_rows_out = splits > 1 ? split_rows : K;
}

void form_split(const GemmArgs &g, int form, int *splits, int *split_rows) {
    skinny_split((int)skinny_grid(g), g.K, form == kSkinnyRowsOfB ? SK_ROWS : KM_BK, splits, split_rows);
}

using RowsKern = void (*)(SkinnyArgs, int);
using KmajKern = void (*)(KmajArgs, int);

bool aligned16(const float *p, int64_t ld) { return reinterpret_cast<uintptr_t>(p) % 16 == 0 && ld % 4 == 0; }

KmajKern kmaj_staged_instance(bool vec, bool tout) {
    if (vec) return tout ? sgemm_kmaj_kernel<true, false, true, 2> : sgemm_kmaj_kernel<true, false, false, 2>;
    return tout ? sgemm_kmaj_kernel<false, false, true, 2> : sgemm_kmaj_kernel<false, false, false, 2>;
}

template <int DEPTH>
KmajKern kmaj_instance(bool vec, bool xt, bool tout) {
    if (vec)
        return xt ? (tout ? sgemm_kmaj_kernel<true, true, true, DEPTH> : sgemm_kmaj_kernel<true, true, false, DEPTH>)
                  : (tout ? sgemm_kmaj_kernel<true, false, true, DEPTH> : sgemm_kmaj_kernel<true, false, false, DEPTH>);
    return xt ? (tout ? sgemm_kmaj_kernel<false, true, true, DEPTH> : sgemm_kmaj_kernel<false, true, false, DEPTH>)
              : (tout ? sgemm_kmaj_kernel<false, false, true, DEPTH> : sgemm_kmaj_kernel<false, false, false, DEPTH>);
}

// The streamed operand W and the small operand X of the K-major forms.
KmajArgs kmaj_args(const GemmArgs &g, int form, float *ws, int splits, int split_rows, bool *xt) {
    const bool bw = form == kSkinnyBKMajor;   // W = B (N x K); else W = A (M x K), D = C transposed
    KmajArgs a;
    a.W = bw ? g.B : g.A;
    a.ldw = bw ? g.ldb : g.lda;
    a.R = bw ? g.N : g.M;
    a.X = bw ? g.A : g.B;
    a.MX = bw ? g.M : g.N;
    a.K = g.K;
    // X given k-major: A stored K x M (TT), or B as given, K x N (NN).
    *xt = bw ? g.trans_a != 0 : g.trans_b == 0;
    const int64_t ldx = bw ? g.lda : g.ldb;
    a.x_si = *xt ? 1 : ldx;
    a.x_sk = *xt ? ldx : 1;
    a.alpha = g.alpha;
    a.beta = g.beta;
    a.C = g.C;
    a.c_si = bw ? g.ldc : 1;
    a.c_sr = bw ? 1 : g.ldc;
    a.ws = ws;
    a.w_si = bw ? g.N : 1;                      // partials in C's order, rows of N
    a.w_sr = bw ? 1 : g.N;
    a.splits = splits;
    a.split_rows = split_rows;
    return a;
}

}  // namespace

int64_t skinny_scratch_bytes(const GemmArgs &g) {
    const int form = skinny_form(g.trans_a, g.trans_b, g.M, g.N, g.K, g.lda, g.ldb);
    if (form < 0) return 0;
    int splits = 1, split_rows = 0;
    form_split(g, form, &splits, &split_rows);
    return splits > 1 ? (int64_t)splits * g.M * g.N * (int64_t)sizeof(float) : 0;
}

hipError_t launch_skinny(const GemmArgs &g, bool vec_loads, hipStream_t stream) {
    const int form = skinny_form(g.trans_a, g.trans_b, g.M, g.N, g.K, g.lda, g.ldb);
    if (form < 0) return hipErrorInvalidValue;
    const int strips = (int)skinny_grid(g);
    int splits = 1, split_rows = 0;
    form_split(g, form, &splits, &split_rows);
    float *ws = nullptr;
    if (splits > 1) {
        hipError_t e = scratch_acquire(g.scratch, (size_t)skinny_scratch_bytes(g), stream,
                                       reinterpret_cast<void **>(&ws));
        if (e != hipSuccess) return e;
    }
    const dim3 grid(strips * splits);
    if (form == kSkinnyRowsOfB) {
        SkinnyArgs sa;
        sa.g = g;
        sa.ws = ws;
        sa.splits = splits;
        sa.split_rows = split_rows;
        // One block of 16 rows of A for M <= 16, two for 16 < M <= 32; three
        // batches in flight on grids of at most kDeepStrips strips.
        const int mb = g.M > 16 ? 2 : 1;
        const int depth = strips <= kDeepStrips ? 3 : 2;
        RowsKern k;
        if (vec_loads)
            k = mb == 2 ? (depth == 3 ? sgemm_skinny_kernel<true, 2, 3> : sgemm_skinny_kernel<true, 2, 2>)
                        : (depth == 3 ? sgemm_skinny_kernel<true, 1, 3> : sgemm_skinny_kernel<true, 1, 2>);
        else
            k = mb == 2 ? (depth == 3 ? sgemm_skinny_kernel<false, 2, 3> : sgemm_skinny_kernel<false, 2, 2>)
                        : (depth == 3 ? sgemm_skinny_kernel<false, 1, 3> : sgemm_skinny_kernel<false, 1, 2>);
        hipLaunchKernelGGL(k, grid, dim3(SK_NT), 0, stream, sa, strips);
    } else {
        bool xt = false;
        const KmajArgs a = kmaj_args(g, form, ws, splits, split_rows, &xt);
        const bool tout = form == kSkinnyAKMajor;
        // 16-byte loads of W, and of X where X is read along k.
        const bool vec = aligned16(a.W, a.ldw) && (xt || aligned16(a.X, a.x_si));
        const bool deep = (int64_t)split_rows >= (int64_t)kDeepBatches * KM_BK * SK_NW;
        // X read along k is staged in LDS when each wave has 2 to 4 batches.
        const bool staged = !xt && split_rows >= 2 * KM_BK * SK_NW && split_rows <= KM_XL_ROWS;
        const KmajKern k = deep ? kmaj_instance<1>(vec, xt, tout)
                                : staged ? kmaj_staged_instance(vec, tout) : kmaj_instance<0>(vec, xt, tout);
        hipLaunchKernelGGL(k, grid, dim3(SK_NT), 0, stream, a, strips);
    }
    hipError_t e = hipGetLastError();
    if (splits > 1) {
        if (e == hipSuccess) {
            const int64_t total = (int64_t)g.M * g.N;
            int64_t blocks = (total + 255) / 256;
            if (blocks > 4096) blocks = 4096;
            hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g, ws, splits);
            e = hipGetLastError();
        }
        const hipError_t r = scratch_release(g.scratch, ws, stream);
        if (e == hipSuccess) e = r;
    }
    return e;
}

}  // namespace sgemm
