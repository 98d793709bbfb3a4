// FP32 GEMM on 256 x 256 tiles, one per CU at a time, for grids whose rounds of
// 256 tiles lie almost entirely inside C; the same kernel on 192 x 192 tiles
// (4 waves of 96 x 96, one work-group per CU, 96 KB of LDS), on 128 x 128
// tiles (4 waves of 64 x 64, two work-groups per CU, 64 KB of LDS each) and on
// 64 x 64 tiles (4 waves of 32 x 32, four work-groups per CU; grids of at most
// one tile per CU run 8 waves per tile, two groups splitting K) serves whole
// grids of those tiles.  The description below is that of the 256 x 256 form.
//
// One work-group per CU, 4 waves of 128 x 128 (4 x 4 blocks of 32x32x2 MFMA,
// 256 accumulators per lane, kept in the accumulation registers): per MFMA a
// wave reads half the fragment bytes of a 64 x 64 wave tile, and per output
// element the operands are read from L2 half as often as with 128 x 128 tiles
// (the larger block tiles of "How a Matmul Kernel Gets Fast", section 9, and
// the warp tiles of its section 13, here one 64-lane wave per sub-tile).
//
// The operands go from memory straight into LDS (buffer_load_dwordx4 with the
// lds flag: each lane's 16 bytes land at the instruction's LDS base + 16 *
// lane), so no registers stage them: slices of 16 k in four LDS stages of
// 32 KB, the loads of slice t+3 issued while slice t is multiplied.  With one
// wave per SIMD nothing else hides a stall, and a wave issues in order, so
// every load, fragment read and address computation is placed right after an
// MFMA, where it goes out while the matrix core works.
//
// Ordering without __syncthreads (its fence would wait for every load in
// flight): at the top of slice t each wave waits until at most the 16 loads
// of slices t+1 and t+2 are outstanding (vector-memory counts complete in
// order) and for its own LDS reads, then joins an s_barrier; past it every
// wave's part of slice t is in LDS and every wave is done with the stage that
// slice t+3 is loaded into.
//
// LDS layouts, per operand and slice (16 KB):
//   rows of k (A as given, B given transposed): 256 rows of 16 floats (64
//   bytes, 4 chunks of 4 floats); chunk c of row x sits at position
//   c ^ ((x >> 2) & 3), which keeps the 16-byte fragment reads free of bank
//   conflicts.  One load instruction fills 16 rows.
//   rows of x (B as given, A given transposed): 16 rows of 256 floats (1 KB,
//   one load instruction each; smaller tiles lay their shorter rows end to
//   end, each instruction filling the next 1 KB); rows 8..15, read by the
//   second half-wave, are rotated by 32 floats so that the two half-waves,
//   which read rows k and k + 8 at the same x, fall in opposite halves of the
//   bank space (every row length here is a multiple of the 64 banks).
//
// Edges.  K, and the x extent of an operand stored along x, are multiples of
// 4, so a 16-byte group never straddles an edge (groups of an operand stored
// along k lie in one row, whole rows past its x edge).  Tiles that cross M or
// N give each group outside M or N an out-of-range lane offset: the load writes zeros to LDS without touching
// memory (adding exact zeros changes no sum).  When K is not a multiple of 16
// the loads of the partial last slice do the same for groups past K; they are
// issued by the last iterations of the slice loop, which run a copy of the loop
// with that check, so the other iterations keep constant offsets.  Tiles that
// cross M or N store through a buffer resource over the valid part of C, whose
// extent drops rows past M and whose out-of-range offsets drop columns past N.
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "gemm_internal.hpp"

namespace sgemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// How an operand is stored: runs along k (A as given, B given transposed) or
// runs along x (B as given, A given transposed), x being M for A and N for B.
enum : int { kKRows = 0, kXRows = 1 };

constexpr int BK = 16;                   // slice depth
constexpr int NT = 256;                  // 4 waves in a 2 x 2 arrangement
constexpr int NST = 4;                   // LDS stages

// Geometry of a TS x TS tile (TS = 256: one work-group per CU; the same
// kernel on 192 x 192 tiles, one work-group per CU, on 128 x 128, two, and on
// 64 x 64, four).
template <int TS>
struct Geo {
    static constexpr int BM = TS, BN = TS;
    static constexpr int WT = TS / 2;             // wave tile
    static constexpr int BLK = WT / 32;           // 32x32 blocks per wave and direction
    static constexpr int PANEL = TS * BK * 4;     // bytes per operand and slice
    static constexpr int STAGE = 2 * PANEL;
    static constexpr int LPO = TS / 64;           // load instructions per wave, operand and slice
    static constexpr int LPS = 2 * LPO;
    static constexpr int XROW = TS * 4;           // bytes of one LDS row of an operand stored along x
    static constexpr int XLANES = TS / 4;         // its 16-byte chunks
    static constexpr int KROWS_W = TS / 4;        // rows of an operand stored along k per wave
    static_assert(NST * STAGE <= 160 * 1024, "LDS");
    static_assert(BK * XROW == 4 * LPO * 1024, "rows of x: the 4 waves' loads fill a panel");
};

__device__ float raw_buffer_load_f32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.f32");
// Vector-memory buffer store: offsets at or past the extent are dropped.
__device__ void raw_buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.store.f32");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, unsigned char *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0, 0);
}

// A lane offset past every resource extent used here (extents stay below
// 2^31 bytes): the load writes zeros to LDS and touches no memory.
constexpr int kOutOfRange = (int)0x80000000u;

// One operand's staging: the per-lane byte offsets of its load instructions
// (from the slice origin), the LDS bytes of each instruction's destination
// (from the panel start), and the slice-origin resource.  EDGE: the tile
// crosses the operand's extent along x (xs valid values of x) or the slice
// crosses K; every group that lies outside gets an out-of-range offset, so
// LDS receives zeros there (adding exact zeros changes no sum).
template <int L, bool EDGE, int TS>
struct Operand {
    using G = Geo<TS>;
    const float *X;      // first element of the tile's x range at k = 0
    int64_t ld;
    int xs, K;
    int off[G::LPO];
    int dst[G::LPO];
    int gx[G::LPO];      // x of the lane's group (rows of k: its row; rows of x: its first column)
    int gk[G::LPO];      // k of the lane's group (rows of k: its first k; rows of x: its row)

    __device__ __forceinline__ Operand(const float *base, int64_t ld_, int x0, int xn, int K_, int wave, int lane)
        : ld(ld_), xs(min(TS, xn - x0)), K(K_) {
        X = L == kKRows ? base + (int64_t)x0 * ld_ : base + x0;
#pragma unroll
        for (int j = 0; j < G::LPO; ++j) {
            if (L == kKRows) {
                // 16 rows of 64 bytes per instruction
                const int x = wave * G::KROWS_W + 16 * j + (lane >> 2);
                const int c = (lane & 3) ^ ((x >> 2) & 3);
                off[j] = (x * (int)ld_ + 4 * c) * 4;
                dst[j] = (wave * G::KROWS_W + 16 * j) * BK * 4;
                gx[j] = x;
                gk[j] = 4 * c;
            } else {
                // The panel's 16 rows of k lie end to end; instruction j of
                // the wave fills its next 1 KB, the lane's 16 bytes at byte
                // b: row k, position p, which holds chunk c (rows 8..15
                // rotated by 32 floats).  Rows of 1 KB or a power-of-two part
                // of it keep whole rows per instruction, in that form.
                int k, p;
                if constexpr (1024 % G::XROW == 0) {
                    const int row0 = (wave * G::LPO + j) * (1024 / G::XROW);
                    k = row0 + lane / G::XLANES;
                    p = lane % G::XLANES;
                    dst[j] = row0 * G::XROW;
                } else {
                    const int b = (wave * G::LPO + j) * 1024 + 16 * lane;
                    k = b / G::XROW;
                    p = b % G::XROW / 16;
                    dst[j] = (wave * G::LPO + j) * 1024;
                }
                const int c = k >= BK / 2 ? (p + 8) % G::XLANES : p;
                off[j] = (k * (int)ld_ + 4 * c) * 4;
                gx[j] = 4 * c;
                gk[j] = k;
            }
        }
    }
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t slice(int k0) const {
        if (L == kKRows) return rsrc(X + k0, (int)(((EDGE ? xs : TS) - 1) * ld + BK) * 4);
        return rsrc(X + (int64_t)k0 * ld, (int)(((BK - 1) * ld + TS) * 4));
    }
    // CK: the slice may reach past K (only the last one does).
    template <bool CK>
    __device__ __forceinline__ int offset(int j, int k0) const {
        if (!EDGE && !CK) return off[j];
        bool ok = true;
        if (EDGE) ok = gx[j] < xs;
        if (CK) ok = ok && k0 + gk[j] < K;
        return ok ? off[j] : kOutOfRange;
    }
};

// Fragment addresses of one operand for the lane: x = xw + 32 b + l % 32; the
// half-wave h = l / 32 owns k = 8 h .. 8 h + 7 of each slice, read in two
// halves j = 0, 1 of four k steps (k = 8 h + 4 j + e, e < 4).
template <int L, int TS>
struct FragAddr {
    using G = Geo<TS>;
    int a[G::BLK];       // rows of k: byte address of the lane's chunk 2 h (chunk 2 h + 1 is a[b] ^ 16)
                         // rows of x: byte address of row 8 h, column x (rotated for h = 1)
    __device__ __forceinline__ FragAddr(int xw, int h, int l32) {
#pragma unroll
        for (int b = 0; b < G::BLK; ++b) {
            const int x = xw + 32 * b + l32;
            if (L == kKRows) a[b] = x * BK * 4 + ((2 * h) ^ ((x >> 2) & 3)) * 16;
            else if ((TS & (TS - 1)) == 0) a[b] = (8 * h) * G::XROW + ((x - 32 * h) & (TS - 1)) * 4;
            else a[b] = (8 * h) * G::XROW + (x - 32 * h + TS) % TS * 4;
        }
    }
};

template <int TS>
struct Frag {
    float a[Geo<TS>::BLK][4];
    float b[Geo<TS>::BLK][4];
};

// Piece q (0 .. 4 + 4 BLK - 1 for one operand of each layout) of the fragment
// reads of half j: for rows of k, piece b reads block b's 16-byte chunk; for
// rows of x, piece 4 b + e reads block b at k step e.
template <int L, int TS>
__device__ __forceinline__ void read_piece(const unsigned char *panel, const FragAddr<L, TS> &fa, int j, int q,
                                           float (&f)[Geo<TS>::BLK][4]) {
    if (L == kKRows) {
        // chunk 2 h + j: positions of chunks 2h and 2h+1 differ in bit 0 of the position only
        const int addr = fa.a[q] ^ (j * 16);
        const f32x4 v = *reinterpret_cast<const f32x4 *>(panel + addr);
        f[q][0] = v[0];
        f[q][1] = v[1];
        f[q][2] = v[2];
        f[q][3] = v[3];
    } else {
        const int b = q >> 2, e = q & 3;
        f[b][e] = *reinterpret_cast<const float *>(panel + fa.a[b] + (4 * j + e) * Geo<TS>::XROW);
    }
}

template <int L, int TS>
constexpr int pieces() { return L == kKRows ? Geo<TS>::BLK : 4 * Geo<TS>::BLK; }

// One TS x TS tile at (m0, n0).  EDGE: the tile crosses M or N.  KG: groups
// of 4 waves that split the tile's K slices between them (KG = 2: waves 4-7
// take the second half of the slices, in LDS stages of their own; both groups
// run the same number of iterations, so every s_barrier is met by all eight
// waves, the group whose range runs past K loading zeros).  At the end the
// second group hands its sums to the first through LDS, which adds them to its
// own (its partial first, so the result does not depend on timing) and writes
// C.  With one work-group per compute unit, the second group doubles the
// MFMA work between two barriers and gives each SIMD a second wave to issue.
// Measured on MI355X (per-launch medians, one group -> two): 1024^3 21.16 ->
// 20.92 µs, 1024 x 1024 x 4096 68.6 -> 66.1 µs; eight LDS stages per group
// instead of four (seven slices in flight) gained nothing on either, and four
// groups (16 waves per CU, 128 registers each) lost: 1024^3 21.9-22.1 against
// 20.9-21.0 µs, slower on every grid of at most one tile per CU tried.
template <int LA, int LB, bool EDGE, int TS, int KG = 1>
__device__ __forceinline__ void big_tile(const GemmArgs &g, int m0, int n0, unsigned char *smem_all) {
    using G = Geo<TS>;
    constexpr int BM = G::BM, BN = G::BN, WT = G::WT, BLK = G::BLK, PANEL = G::PANEL, STAGE = G::STAGE;
    constexpr int LPO = G::LPO, LPS = G::LPS;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wave8 & 3, group = KG > 1 ? wave8 >> 2 : 0;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    unsigned char *smem = smem_all + group * (NST * STAGE);
    // This group's slices: [ks0, ks0 + nk) of the nk_all slices of K.
    const int nk_all = (g.K + BK - 1) / BK;
    const int nk = (nk_all + KG - 1) / KG;
    const int ks0 = group * nk;

    const Operand<LA, EDGE, TS> opa(g.A, g.lda, m0, g.M, g.K, wave, lane);
    const Operand<LB, EDGE, TS> opb(g.B, g.ldb, n0, g.N, g.K, wave, lane);
    auto issue_one = [&](auto ck, int slice, int stage, int i) {
        constexpr bool CK = decltype(ck)::value;
        const int k0 = (ks0 + slice) * BK;
        unsigned char *st = smem + stage * STAGE;
        if (i < LPO) lds_dma16(opa.slice(k0), st + opa.dst[i], opa.template offset<CK>(i, k0));
        else lds_dma16(opb.slice(k0), st + PANEL + opb.dst[i - LPO], opb.template offset<CK>(i - LPO, k0));
    };

    f32x16 acc[BLK][BLK];
#pragma unroll
    for (int i = 0; i < BLK; ++i)
#pragma unroll
        for (int j = 0; j < BLK; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const FragAddr<LA, TS> fra(wm * WT, h, l32);
    const FragAddr<LB, TS> frb(wn * WT, h, l32);
    constexpr int PA = pieces<LA, TS>(), PB = pieces<LB, TS>();
    auto read = [&](const unsigned char *st, int j, int q, Frag<TS> &f) {
        if (q < PA) read_piece<LA, TS>(st, fra, j, q, f.a);
        else read_piece<LB, TS>(st + PANEL, frb, j, q - PA, f.b);
    };
    // MFMA i of a half: k step e = i / BLK^2, block (i / BLK) % BLK, i % BLK.
    auto mfma_one = [&](const Frag<TS> &f, int i) {
        const int e = i / (BLK * BLK), ib = (i / BLK) % BLK, jb = i % BLK;
        acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[ib][e], f.b[jb][e], acc[ib][jb], 0, 0, 0);
    };

    // Slices past the end are loaded again as the last one, into stages that
    // are never read, so every slice issues the same number of loads.
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
#pragma unroll
        for (int i = 0; i < LPS; ++i) issue_one(std::true_type{}, s < nk ? s : nk - 1, s, i);

    Frag<TS> f0, f1;
#pragma unroll
    for (int b = 0; b < BLK; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f1.a[b][e] = 0.f;
            f1.b[b][e] = 0.f;
        }
    constexpr int MF = 4 * BLK * BLK;   // MFMAs per half slice: 64 (TS 256) or 16 (TS 128)
    constexpr int ITEMS = PA + PB + LPS;
    constexpr int PER1 = (ITEMS + MF - 1) / MF, PER2 = (PA + PB + MF - 1) / MF;   // items after each MFMA
    // vmcnt(2 LPS): the loads of slices t+1 and t+2 may stay in flight;
    // lgkmcnt(0); expcnt not waited on (gfx9 encoding: vmcnt bits 3:0 and 15:14).
    constexpr int WAIT = ((2 * LPS) & 15) | (((2 * LPS) >> 4) << 14) | (0 << 8) | (7 << 4);
    //   phase 1: the MFMAs of the previous slice's second half (zeros before
    //            the first slice), each followed by its share of the fragment
    //            reads of this slice's first half and of the loads of slice t+3;
    //   phase 2: the MFMAs of the first half, followed by the reads of the
    //            second half, whose MFMAs are held over to the next slice.
    auto slices = [&](auto ck, int t_begin, int t_end) {
        for (int t = t_begin; t < t_end; ++t) {
            __builtin_amdgcn_s_waitcnt(WAIT);
            __builtin_amdgcn_s_barrier();
            const int ld_slice = t + NST - 1 < nk ? t + NST - 1 : nk - 1;
            const int ld_stage = (t + NST - 1) % NST;
            const unsigned char *st = smem + (t % NST) * STAGE;
#pragma unroll
            for (int i = 0; i < MF; ++i) {
                mfma_one(f1, i);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < PER1; ++u) {
                    const int q = i * PER1 + u;
                    if (q < PA + PB) read(st, 0, q, f0);
                    else if (q < ITEMS) issue_one(ck, ld_slice, ld_stage, q - PA - PB);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < MF; ++i) {
                mfma_one(f0, i);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < PER2; ++u) {
                    const int q = i * PER2 + u;
                    if (q < PA + PB) read(st, 1, q, f1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Iteration t loads slice min(t + 3, nk - 1): the iterations that load a
    // slice reaching past K (the partial last one, or for the second group
    // slices wholly past it) check k, from local slice c - 3 on.
    const int c = (g.K % BK != 0 ? nk_all - 1 : nk_all) - ks0;
    const int t_split = c <= nk - 1 ? max(0, c - (NST - 1)) : nk;
    slices(std::false_type{}, 0, t_split);
    slices(std::true_type{}, t_split, nk);
#pragma unroll
    for (int i = 0; i < MF; ++i) mfma_one(f1, i);
    // Every load issued (including the repeated last slice) has landed before
    // the work-group can end and its LDS be given to another.
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (KG > 1) {
        // Every wave is done with its stages; the second group's sums go
        // through LDS, lane-fastest, to the wave of the first group that owns
        // the same part of the tile.
        static_assert(KG == 2, "two groups");
        constexpr int NACC = BLK * BLK * 16;
        static_assert(4 * NACC * 64 * 4 <= NST * STAGE, "exchange fits one group's stages");
        float *xch = reinterpret_cast<float *>(smem_all) + wave * NACC * 64 + lane;
        __syncthreads();
        if (group == 1) {
#pragma unroll
            for (int ib = 0; ib < BLK; ++ib)
#pragma unroll
                for (int jb = 0; jb < BLK; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) xch[((ib * BLK + jb) * 16 + r) * 64] = acc[ib][jb][r];
        }
        __syncthreads();
        if (group == 1) return;
#pragma unroll
        for (int ib = 0; ib < BLK; ++ib)
#pragma unroll
            for (int jb = 0; jb < BLK; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[ib][jb][r] += xch[((ib * BLK + jb) * 16 + r) * 64];
    }

    // Epilogue in BLK passes of one block row (BLK blocks, 16 BLK values per
    // lane): the C reads of a pass are issued together before its stores
    // (plain stores: with rows of C not 128-byte aligned, non-temporal ones
    // cost 1-6 %).  Accumulator register
    // r of a block holds row 8 (r / 4) + 4 h + r % 4, column l % 32.  Edge
    // tiles go through a buffer resource over the tile's valid part of C: rows
    // past M lie beyond its extent and columns past N get an out-of-range
    // offset, so their loads read zero and their stores are dropped.
    float *Cb = g.C + (int64_t)m0 * g.ldc + n0;
    const float alpha = g.alpha, beta = g.beta;
    const int rows = min(BM, g.M - m0), cols = min(BN, g.N - n0);
    const __amdgpu_buffer_rsrc_t rc = rsrc(Cb, EDGE ? (int)(((int64_t)(rows - 1) * g.ldc + cols) * 4) : 0);
    // Edge offsets: a per-lane part for the block's first row and the lane's
    // column (out of range past N), plus a wave-uniform part for register r.
    auto roff = [&](int r) { return (8 * (r >> 2) + (r & 3)) * (int)g.ldc * 4; };
#pragma unroll
    for (int ib = 0; ib < BLK; ++ib) {
        int cbase[BLK];
#pragma unroll
        for (int jb = 0; jb < BLK; ++jb) {
            const int cc = wn * WT + 32 * jb + l32;
            cbase[jb] = cc < cols ? ((wm * WT + 32 * ib + 4 * h) * (int)g.ldc + cc) * 4 : kOutOfRange;
        }
        float cv[BLK][16];
        if (beta != 0.f) {
#pragma unroll
            for (int jb = 0; jb < BLK; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = wm * WT + 32 * ib + 8 * (r >> 2) + 4 * h + (r & 3);
                    const int cc = wn * WT + 32 * jb + l32;
                    if (EDGE) cv[jb][r] = raw_buffer_load_f32(rc, cbase[jb] + roff(r), 0, 0);
                    else cv[jb][r] = Cb[(int64_t)rr * g.ldc + cc];
                }
        }
#pragma unroll
        for (int jb = 0; jb < BLK; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = wm * WT + 32 * ib + 8 * (r >> 2) + 4 * h + (r & 3);
                const int cc = wn * WT + 32 * jb + l32;
                float v = alpha * acc[ib][jb][r];
                if (beta != 0.f) v = fmaf(beta, cv[jb][r], v);
                if (EDGE) raw_buffer_store_f32(v, rc, cbase[jb] + roff(r), 0, 0);
                else Cb[(int64_t)rr * g.ldc + cc] = v;
            }
    }
}

// Compute units of the current device (cached per device).
hipError_t compute_units(int *out) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return hipSuccess;
        }
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && cus > 0) cache[dev].store(cus, std::memory_order_relaxed);
    *out = cus;
    return hipSuccess;
}

// Work-groups per CU: TS 256 one (256 accumulators per lane), TS 192 one (96
// KB of LDS), TS 128 two, TS 64 four (32 KB of LDS each).
template <int TS>
constexpr int kWavesPerEu = TS == 256 || TS == 192 ? 1 : TS == 128 ? 2 : 4;

template <int LA, int LB, int TS, int KG>
__global__ __launch_bounds__(NT * KG) __attribute__((amdgpu_waves_per_eu(kWavesPerEu<TS>, kWavesPerEu<TS>)))
void sgemm_big_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[KG * NST * Geo<TS>::STAGE];
    static_assert(sizeof(smem) <= 160 * 1024, "LDS");
    poison_lds<sizeof(smem)>(smem);
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * TS, n0 = tn * TS;
    if (m0 + TS > g.M || n0 + TS > g.N) big_tile<LA, LB, true, TS, KG>(g, m0, n0, smem);
    else big_tile<LA, LB, false, TS, KG>(g, m0, n0, smem);
}

// Two groups of waves per tile (KG = 2) when the grid has at most one tile per
// compute unit of the device: on 64 x 64 tiles, and on 128 x 128 tiles with K
// of at least 2048 (there, same box, TFLOP/s, one group -> two: 2048 x 2048 x
// 4096 143.2 -> 145.0, 1024 x 4096 x 4096 143.2 -> 145.3, 4096 x 1024 x 4096
// 143.5 -> 145.3, 2048^3 139.6 -> 140.4; at K = 1024 132.6 -> 131.6).
template <int LA, int LB, int TS>
hipError_t launch(const GemmArgs &g, int group_m, hipStream_t stream) {
    const int tiles_m = (g.M + TS - 1) / TS, tiles_n = (g.N + TS - 1) / TS;
    const int tiles = tiles_m * tiles_n;
    if constexpr (TS == 64 || TS == 128) {
        int cus = 0;
        const hipError_t e = compute_units(&cus);
        if (e != hipSuccess) return e;
        if (tiles <= cus && (TS == 64 || g.K >= 2048)) {
            hipLaunchKernelGGL((sgemm_big_kernel<LA, LB, TS, 2>), dim3(tiles), dim3(2 * NT), 0, stream, g, tiles_m,
                               tiles_n, group_m);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((sgemm_big_kernel<LA, LB, TS, 1>), dim3(tiles), dim3(NT), 0, stream, g, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

// K, and the extent of each operand stored along x (M of A given
// transposed, N of B as given), multiples of 4, so that no 16-byte group
// straddles an edge (an operand stored along k has whole rows past its x
// edge, which read as zeros, so its x extent may be anything); 16-byte
// aligned operands with row strides that are multiples of 4, and operand
// slices that fit the 32-bit buffer offsets.
bool big_tile_fits(const GemmArgs &g) {
    if ((g.trans_a && g.M % 4) || (!g.trans_b && g.N % 4) || g.K % 4 || g.K < 4) return false;
    if (!aligned16(g.A) || !aligned16(g.B) || g.lda % 4 || g.ldb % 4) return false;
    const int64_t lim = (int64_t)1 << 31;
    // (the spans of 256-wide tiles bound those of 128-wide ones)
    auto span = [&](bool krows, int64_t ld) { return krows ? (255 * ld + BK) * 4 : ((BK - 1) * ld + 256) * 4; };
    return span(!g.trans_a, g.lda) < lim && span(g.trans_b, g.ldb) < lim;
}

// Edge tiles address their part of C with 32-bit buffer offsets.
bool big_tile_c_fits(int64_t ldc) { return (255 * ldc + 256) * 4 < ((int64_t)1 << 31); }

int64_t big_tiles(int M, int N) { return (int64_t)((M + 255) / 256) * ((N + 255) / 256); }

namespace {
template <int TS>
hipError_t launch_ts(const GemmArgs &g, int group_m, hipStream_t stream) {
    // A as given has rows of k; B as given has rows of x (N); a transposed
    // operand swaps.
    const bool ta = g.trans_a != 0, tb = g.trans_b != 0;
    if (!ta && !tb) return launch<kKRows, kXRows, TS>(g, group_m, stream);
    if (!ta && tb) return launch<kKRows, kKRows, TS>(g, group_m, stream);
    if (ta && !tb) return launch<kXRows, kXRows, TS>(g, group_m, stream);
    return launch<kXRows, kKRows, TS>(g, group_m, stream);
}
}  // namespace

hipError_t launch_big(const GemmArgs &g, hipStream_t stream) { return launch_ts<256>(g, 4, stream); }

hipError_t launch_dl192(const GemmArgs &g, int group_m, hipStream_t stream) { return launch_ts<192>(g, group_m, stream); }

hipError_t launch_dl128(const GemmArgs &g, int group_m, hipStream_t stream) { return launch_ts<128>(g, group_m, stream); }

hipError_t launch_dl64(const GemmArgs &g, int group_m, hipStream_t stream) { return launch_ts<64>(g, group_m, stream); }

}  // namespace sgemm
