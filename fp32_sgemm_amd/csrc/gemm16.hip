// GEMM with 16-bit inputs (bfloat16 or binary16) on the CDNA4 matrix cores,
// FP32 accumulation and FP32 output: C = alpha * op(A) * op(B) + beta * C.
//
// This is the end point the pages point to once FP32 tiling is exhausted:
// matrix units that take 16-bit inputs and accumulate in FP32, keeping the
// same block tiles, shared-memory staging and pipelining ("Writing a Fast
// Matmul in CUDA, Step by Step", section "Why LLMs use tensor cores instead").
// On gfx950 one v_mfma_f32_32x32x16_{bf16,f16} multiplies a 32x16 by a 16x32
// block: lane l supplies A(l % 32, 8*(l/32) + i) and B(8*(l/32) + i, l % 32)
// for i < 8, eight consecutive k in one 16-byte register group, and returns
// the 32x32 accumulator block in the same layout as the FP32 instruction.
//
// Layout.  The kernel reads both operands as rows of k ("K-major"): A as
// given (M x K) and B given transposed (N x K, the form of a weight matrix
// stored as [out][in]).  Then a lane's eight k are 16 contiguous bytes in
// memory and in LDS, and every fragment is one ds_read_b128.  Other operand
// forms, operands that are not 16-byte aligned, and K not a multiple of the
// 64-deep slice are first packed by pack16_kernel into a K-major copy with K
// padded by zeros (adding exact zeros changes no sum), in the call's scratch
// (a stream-ordered allocation, released after the GEMM kernel).
//
// Tiles.  A work-group computes a 128 x 128 tile of C with 4 waves of 64 x 64
// (2 x 2 blocks of 32 x 32).  Slices of 64 k are staged in LDS, double
// buffered, with two later slices in registers or in flight during the MFMAs
// of the current one, and each k step's fragments read from LDS one step
// ahead of its MFMAs.  A slice row is 128 bytes (8 chunks of 16 bytes); chunk
// c of row r is stored at chunk c ^ ((r >> 1) & 7), so the 16-byte reads of
// eight consecutive rows at one chunk, and the writes of one row's chunks,
// fall in distinct banks.
#include <cstdint>
#include <type_traits>

#include "gemm_internal.hpp"
#include "gemm16_f32.h"

namespace sgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ i32x4 raw_buffer_load_v4i32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.v4i32");
__device__ float raw_buffer_load_f32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.f32");
// Vector-memory buffer store: offsets at or past the extent are dropped.
__device__ void raw_buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.store.f32");
constexpr int kOutOfRange = (int)0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc16(const uint16_t *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, bytes, 0x00020000);
}

constexpr int BM = 128, BN = 128, BK = 64;       // BK in elements
constexpr int NT = 256;
constexpr int ROW_BYTES = BK * 2;                // 128
constexpr int CHUNKS = ROW_BYTES / 16;           // 8
constexpr int A_STAGE = BM * ROW_BYTES;          // bytes
constexpr int B_STAGE = BN * ROW_BYTES;
constexpr int STAGE = A_STAGE + B_STAGE;         // 32 KB
constexpr int LOADS = (BM * CHUNKS) / NT;        // 16-byte groups per thread per operand: 4

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Operand slice addressing: group j of this thread is row (tid / 8) + 32 j,
// chunk tid % 8 of the slice.
struct Loader {
    int off[LOADS];      // byte offsets from the slice origin
    int lds[LOADS];      // byte offsets in the operand's stage
    __device__ __forceinline__ Loader(int64_t ld, int tid) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int r = tid / CHUNKS + (NT / CHUNKS) * j;
            const int c = tid % CHUNKS;
            off[j] = (r * (int)ld + c * 8) * 2;
            lds[j] = r * ROW_BYTES + swz(r, c) * 16;
        }
    }
};

struct Args16 {
    int M, N, K;            // K: multiple of BK (packed or checked)
    float alpha, beta;
    const uint16_t *A;      // M x K, K-major, row stride lda (multiple of 8)
    const uint16_t *B;      // N x K, K-major, row stride ldb; or, for the kernel
                            // that reads B as given, K x N, N-major, row stride ldb
    float *C;
    int64_t lda, ldb, ldc;
    // Direct-to-LDS kernel, K split over work-groups: work-group split s of a
    // tile takes k in [s k_split, (s + 1) k_split) (a multiple of BK) and
    // writes its partial tile at C + s c_split.  Without a split k_split = K
    // and c_split = 0.
    int k_split;
    int64_t c_split;
};

template <bool F16>
__device__ __forceinline__ f32x16 mfma16(i32x4 a, i32x4 b, f32x16 acc) {
    if (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
}

template <bool F16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm16_kernel(Args16 g, int tiles_m,
                                                                                          int tiles_n) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];
    poison_lds<sizeof(smem)>(smem);
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const Loader la(g.lda, tid), lb(g.ldb, tid);
    const int rows_a = min(BM, g.M - m0), rows_b = min(BN, g.N - n0);
    const uint16_t *Ab = g.A + (int64_t)m0 * g.lda;
    const uint16_t *Bb = g.B + (int64_t)n0 * g.ldb;
    // Rows past M (N) lie beyond the resource's extent and read as zeros.
    auto load = [&](int k0, i32x4 (&ra)[LOADS], i32x4 (&rb)[LOADS]) {
        const __amdgpu_buffer_rsrc_t rsa = rsrc16(Ab + k0, (int)(((rows_a - 1) * g.lda + BK) * 2));
        const __amdgpu_buffer_rsrc_t rsb = rsrc16(Bb + k0, (int)(((rows_b - 1) * g.ldb + BK) * 2));
#pragma unroll
        for (int j = 0; j < LOADS; ++j) ra[j] = raw_buffer_load_v4i32(rsa, la.off[j], 0, 0);
#pragma unroll
        for (int j = 0; j < LOADS; ++j) rb[j] = raw_buffer_load_v4i32(rsb, lb.off[j], 0, 0);
    };
    auto store = [&](unsigned char *st, const i32x4 (&ra)[LOADS], const i32x4 (&rb)[LOADS]) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) *reinterpret_cast<i32x4 *>(st + la.lds[j]) = ra[j];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) *reinterpret_cast<i32x4 *>(st + A_STAGE + lb.lds[j]) = rb[j];
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragment rows of this lane: A rows wm*64 + 32 ib + l32, B rows wn*64 + 32 jb + l32.
    int ra_row[2], rb_row[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        ra_row[b] = wm * 64 + 32 * b + l32;
        rb_row[b] = wn * 64 + 32 * b + l32;
    }
    // Fragments of k step s (16 k): one 16-byte read per 32-row block.
    auto read_frags = [&](const unsigned char *st, int s, i32x4 (&fa)[2], i32x4 (&fb)[2]) {
        const int c = 2 * s + h;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            fa[b] = *reinterpret_cast<const i32x4 *>(st + ra_row[b] * ROW_BYTES + swz(ra_row[b], c) * 16);
            fb[b] = *reinterpret_cast<const i32x4 *>(st + A_STAGE + rb_row[b] * ROW_BYTES + swz(rb_row[b], c) * 16);
        }
    };
    // All MFMAs of one slice; the reads of step s+1 are issued before the
    // MFMAs of step s, and issue(s) (global loads of a later slice) runs at the
    // top of step s.
    auto compute = [&](const unsigned char *st, auto issue) {
        i32x4 fa[2][2], fb[2][2];
        read_frags(st, 0, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            issue(s);
            if (s + 1 < BK / 16) read_frags(st, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    acc[ib][jb] = mfma16<F16>(fa[s & 1][ib], fb[s & 1][jb], acc[ib][jb]);
        }
    };
    auto no_issue = [](int) {};
    // Loads of one slice spread over the 4 k steps: 2 of the 8 groups each.
    auto slice_loader = [&](int k0, i32x4 (&ra)[LOADS], i32x4 (&rb)[LOADS]) {
        const __amdgpu_buffer_rsrc_t rsa = rsrc16(Ab + k0, (int)(((rows_a - 1) * g.lda + BK) * 2));
        const __amdgpu_buffer_rsrc_t rsb = rsrc16(Bb + k0, (int)(((rows_b - 1) * g.ldb + BK) * 2));
        return [&, rsa, rsb](int s) {
            ra[s] = raw_buffer_load_v4i32(rsa, la.off[s], 0, 0);
            rb[s] = raw_buffer_load_v4i32(rsb, lb.off[s], 0, 0);
        };
    };

    // Two slices in flight: while slice t is computed from LDS, slice t+1
    // waits in registers for its buffer and slice t+2 is being loaded.  The
    // loads are unconditional (past the end they re-read the last slice, never
    // stored), so the wait counts are the same on every path.
    const int nk = g.K / BK;
    i32x4 ra0[LOADS], rb0[LOADS], ra1[LOADS], rb1[LOADS];
    load(0, ra0, rb0);
    store(smem, ra0, rb0);
    if (nk > 1) load(BK, ra1, rb1);
    __syncthreads();
    int t = 0;
    for (; t + 1 < nk; t += 2) {
        compute(smem, slice_loader((t + 2 < nk ? t + 2 : nk - 1) * BK, ra0, rb0));
        store(smem + STAGE, ra1, rb1);
        __syncthreads();
        compute(smem + STAGE, slice_loader((t + 3 < nk ? t + 3 : nk - 1) * BK, ra1, rb1));
        if (t + 2 < nk) store(smem, ra0, rb0);
        __syncthreads();
    }
    if (t < nk) compute(smem, no_issue);

    // Epilogue: C read in a pass of its own before the stores (see the FP32
    // kernel), elements outside M x N neither read nor written.
    const bool edge = rows_a < BM || rows_b < BN;
    const float alpha = g.alpha, beta = g.beta;
    float cv[2][2][16];
    if (beta != 0.f) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = wm * 64 + 32 * ib + 8 * (r >> 2) + 4 * h + (r & 3);
                    const int cc = wn * 64 + 32 * jb + l32;
                    const bool ok = !edge || (rr < rows_a && cc < rows_b);
                    cv[ib][jb][r] = ok ? g.C[(int64_t)(m0 + rr) * g.ldc + n0 + cc] : 0.f;
                }
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = wm * 64 + 32 * ib + 8 * (r >> 2) + 4 * h + (r & 3);
                const int cc = wn * 64 + 32 * jb + l32;
                if (edge && (rr >= rows_a || cc >= rows_b)) continue;
                float v = alpha * acc[ib][jb][r];
                if (beta != 0.f) v = fmaf(beta, cv[ib][jb][r], v);
                g.C[(int64_t)(m0 + rr) * g.ldc + n0 + cc] = v;
            }
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles for grids that still fill the device: 4 waves of 128 x 128
// (4 x 4 blocks of 32 x 32, 256 accumulators per lane, kept in the
// accumulation registers), one work-group per CU.  Per MFMA a wave reads half
// the fragment bytes of a 64 x 64 wave tile and the slice writes are spread
// over four times the MFMAs, so the LDS traffic (about 96 bytes per clock at
// the MFMA rate, against 128) no longer binds.
// ---------------------------------------------------------------------------
namespace big {
constexpr int BM = 256, BN = 256;
constexpr int WT = 128;                          // wave tile
constexpr int BLK = WT / 32;                     // 4 blocks per wave and direction
}  // namespace big

// Tile geometry of the direct-to-LDS kernel below: TS x TS tiles, 4 waves of
// TS/2 x TS/2, BLK x BLK blocks of 32 x 32 each (TS 256: the tiles above, one
// work-group per CU; TS 192: 3 x 3 blocks, one work-group per CU; TS 128:
// 2 x 2 blocks, two work-groups per CU; the smaller two for grids with too
// few tiles of 256 x 256 to fill the device).
template <int TS>
struct TG {
    static constexpr int BM = TS, BN = TS, WT = TS / 2, BLK = WT / 32;
};

// Epilogue of a TS x TS tile in BLK passes of one block row (BLK blocks, 16
// BLK values per lane): the C reads of a pass are issued together before its
// stores.  Edge tiles go through a buffer resource over the tile's valid part
// of C (rows past M beyond its extent, columns past N out-of-range offsets).
template <int TS>
__device__ __forceinline__ void big_epilogue(const Args16 &g, int m0, int n0, int rows_a, int rows_b, int wm, int wn,
                                             int h, int l32, const f32x16 (&acc)[TG<TS>::BLK][TG<TS>::BLK]) {
    using G = TG<TS>;
    const bool edge = rows_a < G::BM || rows_b < G::BN;
    float *Cb = g.C + (int64_t)m0 * g.ldc + n0;
    const __amdgpu_buffer_rsrc_t rc = rsrc16(reinterpret_cast<const uint16_t *>(Cb),
                                             (int)(((int64_t)(rows_a - 1) * g.ldc + rows_b) * 4));
    const float alpha = g.alpha, beta = g.beta;
    auto pass = [&](int ib, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        float cv[G::BLK][16];
        if (beta != 0.f) {
#pragma unroll
            for (int jb = 0; jb < G::BLK; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = wm * G::WT + 32 * ib + 8 * (r >> 2) + 4 * h + (r & 3);
                    const int cc = wn * G::WT + 32 * jb + l32;
                    cv[jb][r] = EDGE ? raw_buffer_load_f32(rc, cc < rows_b ? (int)((rr * g.ldc + cc) * 4) : kOutOfRange, 0, 0)
                                     : Cb[(int64_t)rr * g.ldc + cc];
                }
        }
#pragma unroll
        for (int jb = 0; jb < G::BLK; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = wm * G::WT + 32 * ib + 8 * (r >> 2) + 4 * h + (r & 3);
                const int cc = wn * G::WT + 32 * jb + l32;
                float v = alpha * acc[ib][jb][r];
                if (beta != 0.f) v = fmaf(beta, cv[jb][r], v);
                if (EDGE) raw_buffer_store_f32(v, rc, cc < rows_b ? (int)((rr * g.ldc + cc) * 4) : kOutOfRange, 0, 0);
                else __builtin_nontemporal_store(v, &Cb[(int64_t)rr * g.ldc + cc]);   // C is not read again here
            }
    };
#pragma unroll
    for (int ib = 0; ib < G::BLK; ++ib) {
        if (edge) pass(ib, std::true_type());
        else pass(ib, std::false_type());
    }
}

// ---------------------------------------------------------------------------
// TS x TS tiles with the operands copied from memory straight into LDS
// (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at the instruction's
// LDS base + 16 * lane, without passing through registers), in slices of 64 k.
// The figures below are those of TS = 256 (one work-group per CU); TS = 192
// and 128 scale every unit and load count by 3/4 and 1/2, and TS = 128 runs
// two work-groups per CU.
//
// A slice row is 128 bytes, one whole cache line (8 chunks of 16), and one
// load instruction fills 1 KB of LDS: 8 rows.  With slices of 32 k (64-byte
// rows, half a line) every line was requested twice from L2: twice
// hipBLASLt's L2 read requests for the same bytes, and the texture unit's
// address queue full for most of the kernel, stalling the load instructions
// and the MFMAs queued behind them.  Chunk c of row r is stored at position
// c ^ ((r >> 1) & 7): the 16 rows that one quarter-wave reads at one chunk
// fill the 64 banks once.  A lane of a load instruction fetches the chunk
// that belongs at its position.
//
// LDS is a ring of five 32 KB units, each holding one operand's slice (160 KB,
// all of it): A of slice s in unit 2s % 5, B in unit (2s + 1) % 5.  While
// slice t is multiplied, units 2t+3 and 2t+4 (mod 5), slice t-1's, are free,
// and the slice issues the loads of B of slice t+1 (into the first, early in
// the slice: it has about one slice of MFMA work to arrive) and of A of slice
// t+2 (into the second, spread over the rest: more than a slice).  Spreading
// the 16 loads of a slice over most of its 64 MFMAs keeps the texture unit's
// queue from filling; with two 64 KB stages, all loads one slice ahead, that
// spread left the last loads too little time.  With one wave per SIMD nothing
// else hides their latency.
//
// Ordering without __syncthreads (whose fence would wait for every load in
// flight): at the top of slice t each wave waits until at most the LPO loads
// of A of slice t+1 (its last-issued ones) are in flight, vector-memory counts
// completing in order, and for its own LDS reads, then joins an s_barrier;
// past it every wave's part of slice t is in LDS and every wave is done with
// slice t-1's units.
//
// B as given (K x N, rows of n; BXM): its slice is kept as it lies in memory,
// 64 rows of k, each 256 n (512 bytes), filled two rows per load instruction,
// row r rotated by 64 * (r % 4) bytes.  A lane's B fragment (eight k at one n)
// then comes from two transposing LDS reads (ds_read_b64_tr_b16): in each
// group of 16 lanes, lanes 4j .. 4j+3 point at 16 consecutive n of row k + j,
// and lane i receives column i of those four rows, four consecutive k at one
// n.  Each half-wave reads 64 bytes of four consecutive rows; the rotation
// puts them in the four quarters of the 64 banks, so a read takes two LDS
// cycles with no conflict (rotating odd rows only, by 64 bytes, left two rows
// on each bank: two conflict cycles per read).  This replaces a packing pass
// over B (one read and one write of all of it).  A given transposed (K x M,
// rows of m; AXM) is staged and read the same way: the MFMA takes its A and B
// fragments in the same lane layout, x standing for m or n.
//
// The compiler cannot tell which LDS bytes a transposing read touches, so it
// makes each one wait for every load into LDS it knows to be in flight
// (vmcnt(0)), which would hold every read until all loads issued so far have
// landed.  The instances with transposing reads therefore issue their loads in
// a form the compiler does not track (lds_dma16_untracked); their order is
// kept by the explicit waits above alone, as it already is for the other
// reads.
// ---------------------------------------------------------------------------
namespace dl {
constexpr int BK = 64;                           // slice depth in elements
constexpr int ROW = BK * 2;                      // 128 bytes
constexpr int NU = 5;                            // units in the ring
constexpr int RPI = 1024 / ROW;                  // K-major rows per load instruction: 8
constexpr int KS = BK / 16;                      // k steps of one MFMA depth: 4
}  // namespace dl

// Ring geometry for TS x TS tiles: a unit holds one operand's slice; a load
// instruction fills 1 KB (8 K-major rows of 128 bytes; along x, the next 1024
// bytes of the wave's rows of k, XROW bytes each, laid end to end).
template <int TS>
struct DLG {
    static constexpr int UNIT = TS * dl::ROW;            // 32, 24 or 16 KB
    static constexpr int LPO = TS / 4 / dl::RPI;         // load instructions per wave and operand per slice
    static constexpr int XROW = TS * 2;                  // along x: one row of k, 512, 384 or 256 bytes
    static constexpr int XCH = XROW / 16;                // its 16-byte chunks
    static_assert(dl::NU * UNIT <= 160 * 1024, "LDS");
    static_assert(dl::BK / 4 * XROW == LPO * 1024, "along x: a wave's 16 rows of k fill its LPO loads");
};

// Along x, row k is rotated by dl_xrot(k) bytes (a multiple of 64) so that the
// four consecutive rows one half-wave's transposing read touches fall in four
// different quarters of the 64 banks: 64 (k % 4) bytes for rows of 512 and 256
// bytes (a multiple of the 256 bank bytes apart), 64 ((k / 2) % 2) for rows of
// 384 (alternately half the banks apart), the only pattern of this form that
// leaves no conflict at every x a read starts at.
template <int TS>
__device__ __forceinline__ int dl_xrot(int k) {
    return TS == 192 ? 64 * ((k >> 1) & 1) : 64 * (k & 3);
}

// Byte offset of an along-x element (row k, column x) in its unit.
template <int TS>
__device__ __forceinline__ int dl_xoff(int k, int x) {
    constexpr int XROW = DLG<TS>::XROW;
    return k * XROW + (x * 2 + dl_xrot<TS>(k)) % XROW;
}

__device__ __forceinline__ int dl_pos(int row, int c) { return c ^ ((row >> 1) & 7); }

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, unsigned char *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0, 0);
}

// The same copy written as one instruction the compiler does not see as a
// memory operation: it inserts no wait for it anywhere, and the caller's own
// s_waitcnt vmcnt counts order it (the hardware counts it like any other
// load).  M0 holds the LDS base, set by the compiler through the constraint;
// one wait state separates that write from the copy.  No register is written.
__device__ __forceinline__ void lds_dma16_untracked(__amdgpu_buffer_rsrc_t rs, unsigned char *lds, int voffset) {
    const unsigned at = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)lds;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rs), "{m0}"(at)
                 : "memory");
}

// Which load of a slice follows MFMA `slot` of k step `phase` (the first BLK
// slots of every step hold fragment reads): 0 .. LPO-1 are B's loads of the
// next slice, one per MFMA from the first free slot on; LPO .. 2 LPO - 1 are
// A's loads of the slice after it, once B's are out (TS 256: one every
// kAStride MFMAs; TS 192: every third; TS 128, 2 free slots per step: one
// per MFMA).  -1: none.
constexpr int kAStride = 4;
template <int TS>
__host__ __device__ constexpr int dl_load_of(int phase, int slot) {
    constexpr int BLK = TG<TS>::BLK, LPO = DLG<TS>::LPO;
    constexpr int per_step = BLK * BLK - BLK;                   // free slots per step
    constexpr int a0 = per_step > LPO ? per_step : LPO;         // A's first position
    constexpr int stride = (4 * per_step - a0) / LPO < kAStride ? (4 * per_step - a0) / LPO : kAStride;
    static_assert(stride >= 1 && a0 + (LPO - 1) * stride < 4 * per_step, "the loads fit the slots");
    if (slot < BLK) return -1;
    const int pos = phase * per_step + (slot - BLK);
    if (pos < LPO) return pos;
    const int a = pos - a0;
    if (a < 0 || a % stride != 0 || a / stride >= LPO) return -1;
    return LPO + a / stride;
}

// Work-groups per CU: one with 256 x 256 tiles (160 KB of LDS) or 192 x 192
// (120 KB), two with 128 x 128 (80 KB each).
template <int TS>
constexpr int kDlPerCu = TS == 128 ? 2 : 1;

template <int TS, bool F16, bool AXM, bool BXM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(kDlPerCu<TS>, kDlPerCu<TS>))) void
gemm16_dl_kernel(Args16 g, int tiles_m, int tiles_n) {
    using G = TG<TS>;
    using D = DLG<TS>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[dl::NU * D::UNIT];
    poison_lds<sizeof(smem)>(smem);
    // Work-group -> (split of K, tile): the splits of one tile are whole
    // grids apart.
    const int tiles = tiles_m * tiles_n;
    const int split = blockIdx.x / tiles;
    int tm, tn;
    tile_of_block(blockIdx.x - split * tiles, tiles_m, tiles_n, TS == 128 ? 8 : 4, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int k0 = split * g.k_split;
    const int tid = threadIdx.x;
    // The wave index is uniform: kept in a scalar register, the LDS bases of
    // the loads need no per-load transfer from a vector register.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int rows_a = min(G::BM, g.M - m0), rows_b = min(G::BN, g.N - n0);
    const uint16_t *Ab = AXM ? g.A + m0 + (int64_t)k0 * g.lda : g.A + (int64_t)m0 * g.lda + k0;
    const uint16_t *Bb = BXM ? g.B + n0 + (int64_t)k0 * g.ldb : g.B + (int64_t)n0 * g.ldb + k0;
    // Any transposing read needs every load into LDS untracked (see above).
    constexpr bool UNTRACKED = AXM || BXM;

    // Load instruction j of this wave covers rows wave*TS/4 + 8 j + lane/8;
    // the lane's position lane % 8 in its row holds chunk dl_pos(row, lane % 8).
    // An operand as given along x (A transposed, K x M; B as given, K x N):
    // the wave's rows of k wave*16 .. wave*16 + 15 lie end to end, and the
    // lane's 16 bytes, byte 1024 j + 16 lane of them, are position p of row
    // k, which holds the chunk that the row's rotation puts there (x past M
    // or N gets an out-of-range offset and arrives as zeros).  Both fill a
    // quarter of their unit per wave.
    auto offsets = [&](bool xm, int64_t ld, int rows, int (&off)[D::LPO]) {
#pragma unroll
        for (int j = 0; j < D::LPO; ++j) {
            if (xm) {
                const int b = 1024 * j + 16 * lane;
                const int k = wave * (dl::BK / 4) + b / D::XROW;
                const int p = b % D::XROW / 16;
                const int cx = (p - dl_xrot<TS>(k) / 16 + D::XCH) % D::XCH;
                off[j] = 8 * cx < rows ? (k * (int)ld + 8 * cx) * 2 : kOutOfRange;
            } else {
                const int r = wave * (G::BM / 4) + dl::RPI * j + (lane >> 3);
                off[j] = (r * (int)ld + dl_pos(r, lane & 7) * 8) * 2;
            }
        }
    };
    int offa[D::LPO], offb[D::LPO];
    offsets(AXM, g.lda, rows_a, offa);
    offsets(BXM, g.ldb, rows_b, offb);
    // Rows past M (N) lie beyond the resource's extent and arrive as zeros.
    auto issue_a = [&](int slice, int unit, int j) {
        unsigned char *dst = smem + unit * D::UNIT + wave * (D::UNIT / 4) + j * 1024;
        if (AXM) {
            const __amdgpu_buffer_rsrc_t rsa =
                rsrc16(Ab + (int64_t)slice * dl::BK * g.lda, (int)(((dl::BK - 1) * g.lda + rows_a) * 2));
            lds_dma16_untracked(rsa, dst, offa[j]);
        } else {
            const __amdgpu_buffer_rsrc_t rsa =
                rsrc16(Ab + slice * dl::BK, (int)(((rows_a - 1) * g.lda + dl::BK) * 2));
            if (UNTRACKED) lds_dma16_untracked(rsa, dst, offa[j]);
            else lds_dma16(rsa, dst, offa[j]);
        }
    };
    auto issue_b = [&](int slice, int unit, int j) {
        unsigned char *dst = smem + unit * D::UNIT + wave * (D::UNIT / 4) + j * 1024;
        if (BXM) {
            const __amdgpu_buffer_rsrc_t rsb =
                rsrc16(Bb + (int64_t)slice * dl::BK * g.ldb, (int)(((dl::BK - 1) * g.ldb + rows_b) * 2));
            lds_dma16_untracked(rsb, dst, offb[j]);
        } else {
            const __amdgpu_buffer_rsrc_t rsb =
                rsrc16(Bb + slice * dl::BK, (int)(((rows_b - 1) * g.ldb + dl::BK) * 2));
            if (UNTRACKED) lds_dma16_untracked(rsb, dst, offb[j]);
            else lds_dma16(rsb, dst, offb[j]);
        }
    };

    f32x16 acc[G::BLK][G::BLK];
#pragma unroll
    for (int i = 0; i < G::BLK; ++i)
#pragma unroll
        for (int j = 0; j < G::BLK; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragment addresses (unit-relative).  K-major: block b of k step s is
    // row x = w*WT + 32 b + l32 of the operand, chunk 2 s + h; the rows of
    // the four blocks differ by 32, which leaves (x >> 1) & 7 alone, so the
    // block only adds 32 rows.  Along x (the MFMA takes A and B fragments of
    // the same shape): the two transposing reads q = 0, 1 of k step s, block
    // b; in lane group g16 = lane / 16 (k half lane / 32, x half g16 % 2),
    // lane 4 j + qq points at row 16 s + 8 h + 4 q + j, x from 32 b +
    // 16 (g16 % 2) + 4 qq of the wave's WT; the step and q only add whole rows.
    int fa_off[dl::KS], fb_off[dl::KS], fax_off[G::BLK], fbx_off[G::BLK];
#pragma unroll
    for (int s = 0; s < dl::KS; ++s) {
        const int pos = dl_pos(l32, 2 * s + h) * 16;
        fa_off[s] = (wm * G::WT + l32) * dl::ROW + pos;
        fb_off[s] = (wn * G::WT + l32) * dl::ROW + pos;
    }
#pragma unroll
    for (int b = 0; b < G::BLK; ++b) {
        const int k = 8 * h + ((lane >> 2) & 3);
        const int xq = 32 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        fax_off[b] = dl_xoff<TS>(k, wm * G::WT + xq);
        fbx_off[b] = dl_xoff<TS>(k, wn * G::WT + xq);
    }
    // Eight k at one x from two transposing reads, four rows apart.
    auto read_tr = [&](const unsigned char *p) {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * D::XROW));
        const i32x2 l2 = __builtin_bit_cast(i32x2, lo), h2 = __builtin_bit_cast(i32x2, hi);
        return i32x4{l2.x, l2.y, h2.x, h2.y};
    };
    auto read_blk = [&](const unsigned char *sa, const unsigned char *sb, int s, int b, i32x4 (&fa)[G::BLK],
                        i32x4 (&fb)[G::BLK]) {
        if (AXM) fa[b] = read_tr(sa + fax_off[b] + 16 * s * D::XROW);
        else fa[b] = *reinterpret_cast<const i32x4 *>(sa + fa_off[s] + 32 * b * dl::ROW);
        if (BXM) fb[b] = read_tr(sb + fbx_off[b] + 16 * s * D::XROW);
        else fb[b] = *reinterpret_cast<const i32x4 *>(sb + fb_off[s] + 32 * b * dl::ROW);
    };
    auto mfma_one = [&](const i32x4 (&fa)[G::BLK], const i32x4 (&fb)[G::BLK], int i) {
        acc[i / G::BLK][i % G::BLK] = mfma16<F16>(fa[i / G::BLK], fb[i % G::BLK], acc[i / G::BLK][i % G::BLK]);
    };

    const int nk = min(g.k_split, g.K - k0) / dl::BK;
    // Before the first slice: A and B of slice 0, A of slice 1 (the last
    // issued, so that slice 0 can start while it is in flight).
#pragma unroll
    for (int j = 0; j < D::LPO; ++j) issue_a(0, 0, j);
#pragma unroll
    for (int j = 0; j < D::LPO; ++j) issue_b(0, 1, j);
    if (nk > 1) {
#pragma unroll
        for (int j = 0; j < D::LPO; ++j) issue_a(1, 2, j);
    }

    // Fragments of the even (x) and odd (y) k steps.
    i32x4 fxa[G::BLK], fxb[G::BLK], fya[G::BLK], fyb[G::BLK];
#pragma unroll
    for (int b = 0; b < G::BLK; ++b) {
        fya[b] = i32x4{0, 0, 0, 0};
        fyb[b] = i32x4{0, 0, 0, 0};
    }
    // One wave per SIMD issues in order, so every other instruction of a
    // slice is placed right after an MFMA and goes out while the matrix core
    // works; sched_barrier keeps the compiler from regrouping them.  Step p of
    // slice t runs the MFMAs of the step before it (for p = 0 the previous
    // slice's last step, zeros before the first slice), each followed by a
    // fragment read of step p or one of the slice's loads.  LB: B of slice
    // t+1 is loaded; LA: A of slice t+2; WAIT8: A of slice t+1 may still be
    // in flight at the top (it is, unless t is the last slice).
    int ua = 0, ub = 1;   // units of slice t: 2t % 5, (2t + 1) % 5
    auto slice = [&](int t, auto wait8_tag, auto lb_tag, auto la_tag) {
        constexpr bool WAIT8 = decltype(wait8_tag)::value;
        constexpr bool LB = decltype(lb_tag)::value;
        constexpr bool LA = decltype(la_tag)::value;
        // vmcnt(LPO) or vmcnt(0), and lgkmcnt(0); expcnt not waited on.
        if (WAIT8) __builtin_amdgcn_s_waitcnt((0 << 14) | (0 << 8) | (7 << 4) | D::LPO);
        else __builtin_amdgcn_s_waitcnt((0 << 14) | (0 << 8) | (7 << 4) | 0);
        __builtin_amdgcn_s_barrier();
        const unsigned char *sa = smem + ua * D::UNIT, *sb = smem + ub * D::UNIT;
        const int unit_b1 = ub + 2 < dl::NU ? ub + 2 : ub + 2 - dl::NU;   // B of slice t+1
        const int unit_a2 = ua + 4 < dl::NU ? ua + 4 : ua + 4 - dl::NU;   // A of slice t+2
        auto step = [&](auto phase_tag, const i32x4 (&ux)[G::BLK], const i32x4 (&uy)[G::BLK],
                        i32x4 (&rx)[G::BLK], i32x4 (&ry)[G::BLK]) {
            constexpr int P = decltype(phase_tag)::value;
#pragma unroll
            for (int i = 0; i < G::BLK * G::BLK; ++i) {
                mfma_one(ux, uy, i);
                __builtin_amdgcn_sched_barrier(0);
                if (i < G::BLK) {
                    read_blk(sa, sb, P, i, rx, ry);
                } else {
                    const int l = dl_load_of<TS>(P, i);
                    if (LB && l >= 0 && l < D::LPO) issue_b(t + 1, unit_b1, l);
                    else if (LA && l >= D::LPO) issue_a(t + 2, unit_a2, l - D::LPO);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        step(std::integral_constant<int, 0>(), fya, fyb, fxa, fxb);
        step(std::integral_constant<int, 1>(), fxa, fxb, fya, fyb);
        step(std::integral_constant<int, 2>(), fya, fyb, fxa, fxb);
        step(std::integral_constant<int, 3>(), fxa, fxb, fya, fyb);
        ua = ua + 2 < dl::NU ? ua + 2 : ua + 2 - dl::NU;
        ub = ub + 2 < dl::NU ? ub + 2 : ub + 2 - dl::NU;
    };
    using yes = std::true_type;
    using no = std::false_type;
    int t = 0;
    for (; t + 2 < nk; ++t) slice(t, yes(), yes(), yes());
    if (t + 1 < nk) {
        slice(t, yes(), yes(), no());
        ++t;
    }
    slice(t, no(), no(), no());
#pragma unroll
    for (int i = 0; i < G::BLK * G::BLK; ++i) mfma_one(fya, fyb, i);

    Args16 gc = g;
    gc.C = g.C + split * g.c_split;
    big_epilogue<TS>(gc, m0, n0, rows_a, rows_b, wm, wn, h, l32, acc);
}

// K-major, K-padded copy of a 16-bit operand: dst[x * Kp + k] = op(x, k) for
// k < K, zero for K <= k < Kp.  XMAJOR: the source holds (x, k) at
// src[k * ld + x] (A given transposed, B as given), and 64 x 64 blocks go
// through LDS so that both the reads (along x) and the writes (along k) are
// contiguous; otherwise at src[x * ld + k].
template <bool XMAJOR>
__global__ __launch_bounds__(256) void pack16_kernel(const uint16_t *src, int64_t ld, int X, int K, uint16_t *dst,
                                                     int Kp) {
    __shared__ uint16_t tile[64][65];
    const int x0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
    if (XMAJOR) {
        for (int kk = ty; kk < 64; kk += 4) {
            const int k = k0 + kk, x = x0 + tx;
            tile[kk][tx] = (k < K && x < X) ? src[(int64_t)k * ld + x] : (uint16_t)0;
        }
        __syncthreads();
        for (int xx = ty; xx < 64; xx += 4) {
            const int x = x0 + xx, k = k0 + tx;
            if (x < X && k < Kp) dst[(int64_t)x * Kp + k] = tile[tx][xx];
        }
    } else {
        for (int xx = ty; xx < 64; xx += 4) {
            const int x = x0 + xx, k = k0 + tx;
            if (x < X && k < Kp) dst[(int64_t)x * Kp + k] = k < K ? src[(int64_t)x * ld + k] : (uint16_t)0;
        }
    }
}

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// A K-major operand can be read in place: 16-byte aligned, row stride a
// multiple of 8 elements, K a multiple of the slice, and 256 rows (the larger
// tile) addressable with 32-bit byte offsets.
bool direct_ok(const void *p, int64_t ld, int K) {
    return aligned16(p) && ld % 8 == 0 && K % BK == 0 && (255 * ld + BK) * 2 < ((int64_t)1 << 31);
}

// An operand along x (B as given, K x N; A transposed, K x M) read in place by
// the direct-to-LDS kernel: 16-byte aligned, row stride and extent (N or M)
// multiples of 8 (a 16-byte group never straddles it), K a multiple of the 64
// the kernels' slices need, and one slice's rows addressable with 32-bit byte
// offsets.
bool direct_xmajor_ok(const void *p, int64_t ld, int N, int K) {
    return aligned16(p) && ld % 8 == 0 && N % 8 == 0 && K % BK == 0 &&
           ((dl::BK - 1) * ld + big::BN) * 2 < ((int64_t)1 << 31);
}

hipError_t pack(const uint16_t *src, int64_t ld, bool xmajor, int X, int K, uint16_t *dst, int Kp,
                hipStream_t stream) {
    const dim3 grid((X + 63) / 64, (Kp + 63) / 64);
    if (xmajor) hipLaunchKernelGGL(pack16_kernel<true>, grid, dim3(256), 0, stream, src, ld, X, K, dst, Kp);
    else hipLaunchKernelGGL(pack16_kernel<false>, grid, dim3(256), 0, stream, src, ld, X, K, dst, Kp);
    return hipGetLastError();
}

// C = alpha * (the splits' partial products, added in split order) + beta * C,
// C read only when beta != 0.  The partials' loads go out eight at a time
// before their additions.
__global__ __launch_bounds__(256) void reduce16_kernel(const float *ws, int splits, int M, int N, float alpha,
                                                       float beta, float *C, int64_t ldc) {
    const int64_t total = (int64_t)M * N;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int sp0 = 0; sp0 < splits; sp0 += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = ws[(int64_t)(sp0 + j < splits ? sp0 + j : splits - 1) * total + t];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (sp0 + j < splits) s += v[j];
        }
        const int64_t i = t / N, jj = t - i * N;
        float *p = C + i * ldc + jj;
        float r = alpha * s;
        if (beta != 0.f) r = fmaf(beta, *p, r);
        *p = r;
    }
}

}  // namespace

// The direct-to-LDS kernel's epilogue addresses a tile of C with 32-bit
// offsets (bounded by a 256-row tile).
bool c_tile_fits(int64_t ldc) { return (255 * ldc + big::BN) * 4 < ((int64_t)1 << 31); }

namespace {

// Time per unit of K of one tile size's grid, from measurement (bf16, beta 0,
// nanoseconds per k): `slots` work-groups run at once (256 CUs times the
// work-groups per CU); each whole round costs `full`; a last partial round
// costs `alone` while it fills at most `knee` of the slots (its tiles run at
// the speed of a CU with little contention for memory, and the rate of one
// tile does not depend on how many others run), rising linearly to `full`.
struct RingCost {
    int slots;
    double full, alone, knee;
    double of(int64_t tiles) const {
        const int64_t rem = tiles % slots;
        double t = (double)(tiles / slots) * full;
        if (rem > 0) {
            const double fill = (double)rem / slots;
            t += fill <= knee ? alone : alone + (full - alone) * (fill - knee) / (1.0 - knee);
        }
        return t;
    }
};

}  // namespace

// Tile size of the direct-to-LDS kernel: the one with the least estimated
// time (ties to the larger tile).
int gemm16_ring_tile(int M, int N) {
    auto tiles = [&](int ts) { return (int64_t)((M + ts - 1) / ts) * ((N + ts - 1) / ts); };
    const double t256 = RingCost{256, 25.7, 19.5, 0.6}.of(tiles(256));
    const double t192 = RingCost{256, 15.0, 12.7, 0.5}.of(tiles(192));
    const double t128 = RingCost{512, 14.7, 10.5, 0.5}.of(tiles(128));
    if (t256 <= t192 && t256 <= t128) return 256;
    return t192 <= t128 ? 192 : 128;
}

// K split of a 128 x 128 grid of fewer than 128 tiles: splits of at least
// kSplit16MinK of K each, about one work-group per CU in all, and at most as
// many as keep the partial products (written once, read once) within half
// the operands' bytes.  Same-box microseconds, bf16 NT, beta 0, no split ->
// this rule (a first rule with up to two work-groups per CU and partials up
// to the operands' bytes in brackets): 16 x 4096 x 4096 33.3 -> 12.4 (13.2);
// 1 x 4096 x 4096 31.2 -> 12.2; 16 x 8192 x 8192 56.1 -> 26.1 (26.2); 64 x
// 4096 x 4096 33.9 -> 14.7 (16.9); 128 x 4096 x 4096 34.3 -> 18.0 (24.1); 256
// x 4096 x 4096 34.0 -> 21.9 (33.5); 256 x 256 x 4096 23.1 -> 11.8 (11.6);
// 128 x 8192 x 4096 -> 22.9 (29.0); 512 x 1024 x 4096 -> 19.9 (33.6).  torch's
// mm of the same operands took 24-29 us on each.
constexpr int kSplit16Slots = 256;
constexpr int kSplit16MinK = 256;
int gemm16_splits(int M, int N, int Kp) {
    const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    if (tiles >= kSplit16Slots / 2) return 1;
    int64_t splits = (kSplit16Slots + tiles - 1) / tiles;
    if (splits > Kp / kSplit16MinK) splits = Kp / kSplit16MinK;
    const int64_t cap = ((int64_t)M + N) * Kp * 2 / ((int64_t)2 * M * N * 4);
    if (splits > cap) splits = cap;
    if (splits < 2) return 1;
    return (int)splits;
}

int64_t gemm16_grid(int M, int N) { return (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

int64_t gemm16_workspace_bytes(int ta, int tb, int M, int N, int K, const void *A, int64_t lda, const void *B,
                               int64_t ldb, bool axm, bool bxm) {
    const int64_t Kp = (int64_t)(K + BK - 1) / BK * BK;
    int64_t bytes = 0;
    if (!axm && (ta || !direct_ok(A, lda, K))) bytes += ((int64_t)M * Kp * 2 + 255) / 256 * 256;
    if (!bxm && (!tb || !direct_ok(B, ldb, K))) bytes += ((int64_t)N * Kp * 2 + 255) / 256 * 256;
    return bytes;
}

hipError_t launch_gemm16(int kind, const GemmArgs &g16, hipStream_t stream) {
    const int ta = g16.trans_a, tb = g16.trans_b;
    const void *A = g16.A, *B = g16.B;
    const int M = g16.M, N = g16.N, K = g16.K;
    const int Kp = (K + BK - 1) / BK * BK;
    // The direct-to-LDS kernel, its tile size from gemm16_ring_tile; the
    // register-staged 128 x 128 kernel only when C's stride is too wide for
    // the former's 32-bit tile offsets.
    const bool ring = c_tile_fits(g16.ldc);
    // Operands along x (A transposed, B as given) are read in place by the
    // direct-to-LDS kernel when they allow it, packed otherwise.
    const bool axm = ta && ring && direct_xmajor_ok(A, g16.lda, M, K);
    const bool bxm = !tb && ring && direct_xmajor_ok(B, g16.ldb, N, K);
    const bool pa = !axm && (ta || !direct_ok(A, g16.lda, K));
    const bool pb = !bxm && (!tb || !direct_ok(B, g16.ldb, K));
    Args16 a;
    a.M = M; a.N = N; a.K = Kp;
    a.alpha = g16.alpha; a.beta = g16.beta;
    a.C = g16.C; a.ldc = g16.ldc;
    a.A = static_cast<const uint16_t *>(A); a.lda = g16.lda;
    a.B = static_cast<const uint16_t *>(B); a.ldb = g16.ldb;
    a.k_split = Kp;
    a.c_split = 0;
    // Tile size, and a K split for small 128 x 128 grids (the partial tiles
    // go to the call's scratch, after any packed operands).
    const int ts = ring ? gemm16_ring_tile(M, N) : 0;
    int splits = ts == 128 && c_tile_fits(N) ? gemm16_splits(M, N, Kp) : 1;
    if (splits > 1) {
        a.k_split = (Kp / splits + BK - 1) / BK * BK;
        splits = (Kp + a.k_split - 1) / a.k_split;
    }
    const int64_t pack_bytes = pa || pb ? gemm16_workspace_bytes(ta, tb, M, N, K, A, g16.lda, B, g16.ldb, axm, bxm) : 0;
    const int64_t part_bytes = splits > 1 ? (int64_t)splits * M * N * 4 : 0;
    void *ws = nullptr;
    if (pack_bytes + part_bytes > 0) {
        hipError_t e = scratch_acquire(g16.scratch, (size_t)(pack_bytes + part_bytes), stream, &ws);
        if (e != hipSuccess) return e;
    }
    float *partials = nullptr;
    if (splits > 1) {
        partials = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + pack_bytes);
        a.C = partials;
        a.ldc = N;
        a.alpha = 1.f;
        a.beta = 0.f;
        a.c_split = (int64_t)M * N;
    }
    if (pa || pb) {
        hipError_t e;
        unsigned char *p = static_cast<unsigned char *>(ws);
        if (pa) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(p);
            e = pack(static_cast<const uint16_t *>(A), g16.lda, ta != 0, M, K, dst, Kp, stream);
            if (e != hipSuccess) {
                (void)scratch_release(g16.scratch, ws, stream);
                return e;
            }
            a.A = dst;
            a.lda = Kp;
            p += ((int64_t)M * Kp * 2 + 255) / 256 * 256;
        }
        if (pb) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(p);
            // B as given is K x N: (n, k) at B[k * ldb + n], M/N-major.
            e = pack(static_cast<const uint16_t *>(B), g16.ldb, tb == 0, N, K, dst, Kp, stream);
            if (e != hipSuccess) {
                (void)scratch_release(g16.scratch, ws, stream);
                return e;
            }
            a.B = dst;
            a.ldb = Kp;
        }
    }
    hipError_t e;
    if (ring) {
        auto go = [&](auto tsc, auto f16, auto ax, auto bx) {
            constexpr int TS = decltype(tsc)::value;
            const int tiles_m = (M + TS - 1) / TS, tiles_n = (N + TS - 1) / TS;
            hipLaunchKernelGGL(
                (gemm16_dl_kernel<TS, decltype(f16)::value, decltype(ax)::value, decltype(bx)::value>),
                dim3(tiles_m * tiles_n * splits), dim3(NT), 0, stream, a, tiles_m, tiles_n);
        };
        auto pick_b = [&](auto ts, auto f16, auto ax) {
            if (bxm) go(ts, f16, ax, std::true_type());
            else go(ts, f16, ax, std::false_type());
        };
        auto pick_a = [&](auto ts, auto f16) {
            if (axm) pick_b(ts, f16, std::true_type());
            else pick_b(ts, f16, std::false_type());
        };
        auto pick_f = [&](auto ts) {
            if (kind == GEMM16_F32_F16) pick_a(ts, std::true_type());
            else pick_a(ts, std::false_type());
        };
        if (ts == 256) pick_f(std::integral_constant<int, 256>());
        else if (ts == 192) pick_f(std::integral_constant<int, 192>());
        else pick_f(std::integral_constant<int, 128>());
        e = hipGetLastError();
        if (e == hipSuccess && splits > 1) {
            const int64_t total = (int64_t)M * N;
            int64_t blocks = (total + 255) / 256;
            if (blocks > 4096) blocks = 4096;
            hipLaunchKernelGGL(reduce16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, partials, splits, M, N,
                               g16.alpha, g16.beta, g16.C, (int64_t)g16.ldc);
            e = hipGetLastError();
        }
    } else {
        const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
        const dim3 grid(tiles_m * tiles_n);
        if (kind == GEMM16_F32_F16)
            hipLaunchKernelGGL(gemm16_kernel<true>, grid, dim3(NT), 0, stream, a, tiles_m, tiles_n);
        else
            hipLaunchKernelGGL(gemm16_kernel<false>, grid, dim3(NT), 0, stream, a, tiles_m, tiles_n);
        e = hipGetLastError();
    }
    const hipError_t r = scratch_release(g16.scratch, ws, stream);
    return e == hipSuccess ? r : e;
}

}  // namespace sgemm

extern "C" int gemm16_f32(int in_type, int trans_a, int trans_b, int M, int N, int K, float alpha, const void *A,
                          int lda, const void *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    if (in_type != GEMM16_F32_BF16 && in_type != GEMM16_F32_F16) return GEMM16_F32_ERR_TYPE;
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return 23;
    if (M < 0) return 1;
    if (N < 0) return 2;
    if (K < 0) return 3;
    const auto one = [](int v) { return v > 1 ? v : 1; };
    const bool need_ab = M > 0 && N > 0 && K > 0 && alpha != 0.f;
    if (need_ab && A == nullptr) return 5;
    if (lda < one(trans_a ? M : K)) return 6;
    if (need_ab && B == nullptr) return 7;
    if (ldb < one(trans_b ? K : N)) return 8;
    if (M > 0 && N > 0 && C == nullptr) return 10;
    if (ldc < one(N)) return 11;
    if (M == 0 || N == 0) return 0;
    sgemm::GemmArgs g;
    g.M = M; g.N = N; g.K = K;
    g.alpha = alpha; g.beta = beta;
    g.A = static_cast<const float *>(A);    // carried as raw pointers; read as 16-bit
    g.B = static_cast<const float *>(B);
    g.C = C;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc;
    g.trans_a = trans_a; g.trans_b = trans_b;
    hipError_t e;
    if (alpha == 0.f || K == 0) {
        e = sgemm::launch_scale_c(g, stream);
        return e == hipSuccess ? 0 : -static_cast<int>(e);
    }
    if (reinterpret_cast<uintptr_t>(A) % 2 || reinterpret_cast<uintptr_t>(B) % 2) return GEMM16_F32_ERR_ALIGN;
    if (K > 4000000 || sgemm::gemm16_grid(M, N) > 0x7fffffff) return 22;
    e = sgemm::launch_gemm16(in_type, g, stream);
    return e == hipSuccess ? 0 : -static_cast<int>(e);
}
