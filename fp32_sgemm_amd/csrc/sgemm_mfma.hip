// FP32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// One work-group computes a BM x BN tile of C.  Its waves each own a WM x WN
// sub-tile held as (WM/32) x (WN/32) blocks of 32x32 FP32 accumulators.  The
// reduction dimension is walked in slices of BK: each slice of A (BM x BK) and
// B (BK x BN) is staged once in LDS and then read by every wave of the group.
// That is the shared-memory tiling of "Learn: Optimizing GEMM" section 5 and
// "How a Matmul Kernel Gets Fast" section 6, the per-thread register tile of
// their sections 6 and 9 (here the accumulator block of an MFMA), and the
// warp-level tiling of "How a Matmul Kernel Gets Fast" section 13 (here one
// 64-lane wave per sub-tile).
//
// Staging.  Global loads are 16-byte (global_load_dwordx4) where the operands
// are 16-byte aligned with row strides that are multiples of 4, four-byte loads
// otherwise.  The loads of slice t+1 are issued into registers before the
// matrix-core work on slice t and written to the other of two LDS buffers after
// it, so one barrier per slice separates producers from consumers (the double
// buffering of "Writing a Fast Matmul in CUDA, Step by Step", section "Bank
// conflicts and double buffering").
//
// LDS layouts.  A 32x32x2 MFMA takes, in lane l, A(l % 32, k) and B(k, l % 32)
// for one of two k values picked by l / 32.  Inside a slice the kernel assigns
// lane half h = l / 32 the k range [h*BK/2, (h+1)*BK/2), so a lane walks a
// contiguous run of k for a fixed row of A.  A is therefore kept K-major in LDS
// exactly as it sits in memory (row stride BK + 4 floats, so the 16-byte reads
// of 16 consecutive rows fall in distinct banks) and read with ds_read_b128,
// four k steps per read.  B is kept N-major as in memory and read with
// ds_read_b32: the two half-waves read rows k and k + BK/2, and the second half
// of the slice's rows is shifted by 32 floats so those two rows sit in opposite
// halves of the bank space.
//
// Edges.  Tiles that cross the M or N edge and the last slice when K is not a
// multiple of BK load through a guarded path that writes zeros for elements
// outside the matrices (adding exact zeros changes no sum), and edge tiles mask
// their stores.  The choice between guarded and plain loads is uniform across
// the work-group, so no barrier sits under divergent control flow.
//
// Epilogue.  C = alpha * acc + beta * C, where C is read only when beta != 0.
#include "gemm_internal.hpp"

namespace sgemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// 16-byte buffer load: base and extent come from a buffer resource in scalar
// registers, the per-lane part is one 32-bit byte offset.  Accesses at or past
// the resource's extent return zeros instead of touching memory.
__device__ f32x4v raw_buffer_load_v4f32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.v4f32");
__device__ float raw_buffer_load_f32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.f32");

// A lane offset past every resource extent used here (extents stay below
// 2^31 bytes): the load returns zero and touches no memory.
constexpr int kOutOfRange = (int)0x80000000u;

// Buffer resource over [base, base + bytes): raw (untyped) access with the
// 32-bit data format, so every lane's offset is checked against `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes, 0x00020000);
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, int PF_ = 1>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int PF = PF_;             // slices loaded ahead of the one being computed
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = (BM / WM) * WAVES_N * 64;
    static constexpr int MB = WM / 32;          // 32x32 accumulator blocks per wave, along M
    static constexpr int NB = WN / 32;          // ... along N
    static constexpr int HALF = BK / 2;         // k values per lane half in one slice
    static constexpr int LDA_S = BK + 4;        // LDS row stride of the A slice (floats)
    static constexpr int B_SHIFT = 32;          // offset of B rows [HALF, BK) in LDS
    static constexpr int A_STAGE = BM * LDA_S;
    static constexpr int B_STAGE = BK * BN + B_SHIFT;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int A_VECS = BM * BK / 4 / NT;   // 4-float groups per thread per slice
    static constexpr int B_VECS = BK * BN / 4 / NT;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert((BM * BK) % (4 * NT) == 0 && (BK * BN) % (4 * NT) == 0, "load split");
    static_assert(2 * STAGE * 4 <= 160 * 1024, "LDS");
};

// Per-thread addressing of the 4-float groups a thread stages for every slice:
// group i of A is row ar[i], columns ac[i]..ac[i]+3 of the slice; group i of B
// is row br[i], columns bc[i]..bc[i]+3.  The row pointers (guarded loads) and
// the byte offsets from the slice origin (buffer loads of interior slices) are
// formed once.
template <class T>
struct Stager {
    const float *pa[T::A_VECS];
    const float *pb[T::B_VECS];
    int ar[T::A_VECS], ac[T::A_VECS];
    int br[T::B_VECS], bc[T::B_VECS];
    int oa[T::A_VECS], ob[T::B_VECS];

    __device__ __forceinline__ Stager(const GemmArgs &g, int m0, int n0, int tid) {
#pragma unroll
        for (int i = 0; i < T::A_VECS; ++i) {
            const int q = tid + i * T::NT;
            ar[i] = q / (T::BK / 4);
            ac[i] = (q % (T::BK / 4)) * 4;
            pa[i] = g.A + (int64_t)(m0 + ar[i]) * g.lda + ac[i];
            oa[i] = (ar[i] * (int)g.lda + ac[i]) * 4;
        }
#pragma unroll
        for (int i = 0; i < T::B_VECS; ++i) {
            const int q = tid + i * T::NT;
            br[i] = q / (T::BN / 4);
            bc[i] = (q % (T::BN / 4)) * 4;
            pb[i] = g.B + (int64_t)br[i] * g.ldb + n0 + bc[i];
            ob[i] = (br[i] * (int)g.ldb + bc[i]) * 4;
        }
    }
};

template <bool VEC>
__device__ __forceinline__ float4 ld4(const float *p) {
    if (VEC) return *reinterpret_cast<const float4 *>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}

// Loads 4-float group p of the slice starting at column k0 of A / row k0 of
// B: groups 0 .. A_VECS-1 are A's, the rest B's.  GMN: the tile crosses the M
// or N edge, so rows of A beyond M and columns of B beyond N read as zero.
// GK: the slice crosses the K edge, so k >= K reads as zero.  Nothing outside
// the matrices is accessed.
// Resources over the A and B elements of the slice at k0 that lie inside the
// matrices: the rows of A below M, and B up to its last valid column in the
// slice's last row.  A rows past M therefore read as zeros by themselves; B
// columns past N need an out-of-range lane offset (load_part).
struct SliceRsrc {
    __amdgpu_buffer_rsrc_t a, b;
};

template <class T>
__device__ __forceinline__ SliceRsrc slice_rsrc(const GemmArgs &g, int m0, int n0, int k0) {
    const int rows = min(T::BM, g.M - m0);
    const int cols = min(T::BN, g.N - n0);
    SliceRsrc r;
    r.a = make_rsrc(g.A + (int64_t)m0 * g.lda + k0, (int)(((rows - 1) * g.lda + T::BK) * 4));
    r.b = make_rsrc(g.B + (int64_t)k0 * g.ldb + n0, (int)(((T::BK - 1) * g.ldb + cols) * 4));
    return r;
}

// Slices that do not cross the K edge are loaded with 16-byte buffer loads
// when VEC; the K-edge slice (GK) and 4-byte loads go through row pointers.
template <class T, bool VEC, bool GMN, bool GK>
__device__ __forceinline__ void load_part(const GemmArgs &g, const Stager<T> &s, int m0, int n0, int k0,
                                          const SliceRsrc &r, int p, float4 (&ra)[T::A_VECS],
                                          float4 (&rb)[T::B_VECS]) {
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr bool BUF = VEC && !GK;
    if (p < T::A_VECS) {
        const int i = p;
        const float *ptr = s.pa[i] + k0;
        const bool row_ok = !GMN || (m0 + s.ar[i] < g.M);
        if (BUF) {
            const f32x4v v = raw_buffer_load_v4f32(r.a, s.oa[i], 0, 0);
            ra[i] = make_float4(v[0], v[1], v[2], v[3]);
        } else if (!GK) {
            ra[i] = row_ok ? ld4<VEC>(ptr) : zero;
        } else {
            const int k = k0 + s.ac[i];
            float4 v = zero;
            if (row_ok) {
                if (k + 0 < g.K) v.x = ptr[0];
                if (k + 1 < g.K) v.y = ptr[1];
                if (k + 2 < g.K) v.z = ptr[2];
                if (k + 3 < g.K) v.w = ptr[3];
            }
            ra[i] = v;
        }
    } else {
        const int i = p - T::A_VECS;
        const float *ptr = s.pb[i] + (int64_t)k0 * g.ldb;
        const bool row_ok = !GK || (k0 + s.br[i] < g.K);
        if (BUF) {
            const int n = n0 + s.bc[i];
            const int off = (!GMN || n + 3 < g.N) ? s.ob[i] : kOutOfRange;
            const f32x4v v = raw_buffer_load_v4f32(r.b, off, 0, 0);
            float4 w = make_float4(v[0], v[1], v[2], v[3]);
            if (GMN && n < g.N && n + 3 >= g.N) {
                // The group straddles column N (only when N is not a multiple of 4).
                w.x = raw_buffer_load_f32(r.b, s.ob[i], 0, 0);
                w.y = raw_buffer_load_f32(r.b, n + 1 < g.N ? s.ob[i] + 4 : kOutOfRange, 0, 0);
                w.z = raw_buffer_load_f32(r.b, n + 2 < g.N ? s.ob[i] + 8 : kOutOfRange, 0, 0);
                w.w = 0.f;
            }
            rb[i] = w;
        } else if (!GMN) {
            rb[i] = row_ok ? ld4<VEC>(ptr) : zero;
        } else {
            const int n = n0 + s.bc[i];
            float4 v = zero;
            if (row_ok) {
                if (VEC && n + 3 < g.N) {
                    v = ld4<true>(ptr);
                } else {
                    if (n + 0 < g.N) v.x = ptr[0];
                    if (n + 1 < g.N) v.y = ptr[1];
                    if (n + 2 < g.N) v.z = ptr[2];
                    if (n + 3 < g.N) v.w = ptr[3];
                }
            }
            rb[i] = v;
        }
    }
}

template <class T, bool VEC, bool GMN, bool GK>
__device__ __forceinline__ void load_slice(const GemmArgs &g, const Stager<T> &s, int m0, int n0, int k0,
                                           float4 (&ra)[T::A_VECS], float4 (&rb)[T::B_VECS]) {
    const SliceRsrc r = slice_rsrc<T>(g, m0, n0, k0);
#pragma unroll
    for (int p = 0; p < T::A_VECS + T::B_VECS; ++p) load_part<T, VEC, GMN, GK>(g, s, m0, n0, k0, r, p, ra, rb);
}

template <class T>
__device__ __forceinline__ void store_slice(float *stage, int tid,
                                            const float4 (&ra)[T::A_VECS],
                                            const float4 (&rb)[T::B_VECS]) {
    float *As = stage;
    float *Bs = stage + T::A_STAGE;
#pragma unroll
    for (int i = 0; i < T::A_VECS; ++i) {
        const int q = tid + i * T::NT;
        const int r = q / (T::BK / 4), c = (q % (T::BK / 4)) * 4;
        *reinterpret_cast<float4 *>(As + r * T::LDA_S + c) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < T::B_VECS; ++i) {
        const int q = tid + i * T::NT;
        const int r = q / (T::BN / 4), c = (q % (T::BN / 4)) * 4;
        *reinterpret_cast<float4 *>(Bs + r * T::BN + (r >= T::HALF ? T::B_SHIFT : 0) + c) = rb[i];
    }
}

// Fragments of one chunk (4 k steps) of a slice: for each 32-row block of the
// wave's A sub-tile one float4 (4 consecutive k of this lane's row), and for
// each 32-column block of B four values (the same 4 k, this lane's column).
template <class T>
struct Frag {
    float4 a[T::MB];
    float b[T::NB][4];
};

template <class T>
__device__ __forceinline__ void read_frag(const float *As, const float *Bs, int c, Frag<T> &f) {
#pragma unroll
    for (int ib = 0; ib < T::MB; ++ib)
        f.a[ib] = *reinterpret_cast<const float4 *>(As + ib * 32 * T::LDA_S + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int jb = 0; jb < T::NB; ++jb)
            f.b[jb][e] = Bs[(4 * c + e) * T::BN + jb * 32];
}

template <class T>
__device__ __forceinline__ void mfma_frag(const Frag<T> &f, f32x16 (&acc)[T::MB][T::NB]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
            for (int jb = 0; jb < T::NB; ++jb) {
                const float av = e == 0 ? f.a[ib].x : e == 1 ? f.a[ib].y : e == 2 ? f.a[ib].z : f.a[ib].w;
                acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, f.b[jb][e], acc[ib][jb], 0, 0, 0);
            }
}

// All MFMAs of one slice.  The LDS reads of chunk c+1 are issued before the
// MFMAs of chunk c, so their latency hides behind matrix-core work.  `issue(c)`
// runs at the top of chunk c; the K loop uses it to spread the global loads of
// a later slice over the slice's MFMAs instead of issuing them in one burst.
struct NoIssue {
    __device__ __forceinline__ void operator()(int) const {}
};

template <class T, class Issue>
__device__ __forceinline__ void compute_slice(const float *stage, int wm, int wn, int lane,
                                              f32x16 (&acc)[T::MB][T::NB], const Issue &issue) {
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const float *As = stage + (wm * T::WM + l32) * T::LDA_S + h * T::HALF;
    const float *Bs = stage + T::A_STAGE + h * (T::HALF * T::BN + T::B_SHIFT) + wn * T::WN + l32;
    constexpr int CH = T::HALF / 4;
    Frag<T> f[2];
    read_frag<T>(As, Bs, 0, f[0]);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        issue(c);
        if (c + 1 < CH) read_frag<T>(As, Bs, c + 1, f[(c + 1) & 1]);
        // Keep the compiler from sinking those reads below the MFMAs.
        __builtin_amdgcn_sched_barrier(0);
        mfma_frag<T>(f[c & 1], acc);
    }
}

template <class T>
__device__ __forceinline__ void compute_slice(const float *stage, int wm, int wn, int lane,
                                              f32x16 (&acc)[T::MB][T::NB]) {
    compute_slice<T>(stage, wm, wn, lane, acc, NoIssue());
}

// The K loop of one tile.  Slices are processed in the order: the partial
// slice at the K edge first (when K is not a multiple of BK), then the full
// slices from k = 0 up, so only the first slice ever needs the K guard.
template <class T, bool VEC, bool GMN>
__device__ __forceinline__ void k_loop(const GemmArgs &g, int m0, int n0, int tid, int wm, int wn,
                                       int lane, float *smem, f32x16 (&acc)[T::MB][T::NB]) {
    const Stager<T> s(g, m0, n0, tid);
    const int nkf = g.K / T::BK;
    const bool tail = nkf * T::BK != g.K;
    const int nk = nkf + (tail ? 1 : 0);
    // k0 of the slice processed at position idx >= 1 (position 0 is the tail
    // slice when there is one).
    const int shift = tail ? 1 : 0;
    auto k0_of = [&](int idx) { return (idx - shift) * T::BK; };

    if (T::PF == 1) {
        float4 ra[T::A_VECS], rb[T::B_VECS];
        if (tail) load_slice<T, VEC, GMN, true>(g, s, m0, n0, nkf * T::BK, ra, rb);
        else load_slice<T, VEC, GMN, false>(g, s, m0, n0, 0, ra, rb);
        store_slice<T>(smem, tid, ra, rb);
        __syncthreads();
        for (int t = 0; t < nk; ++t) {
            const bool more = t + 1 < nk;
            if (more) load_slice<T, VEC, GMN, false>(g, s, m0, n0, k0_of(t + 1), ra, rb);
            compute_slice<T>(smem + (t & 1) * T::STAGE, wm, wn, lane, acc);
            if (more) store_slice<T>(smem + ((t + 1) & 1) * T::STAGE, tid, ra, rb);
            __syncthreads();
        }
    } else {
        // Two register sets: while slice t is computed from LDS, slice t+1
        // waits in registers for its LDS buffer and slice t+2 is in flight.
        float4 ra0[T::A_VECS], rb0[T::B_VECS], ra1[T::A_VECS], rb1[T::B_VECS];
        if (tail) load_slice<T, VEC, GMN, true>(g, s, m0, n0, nkf * T::BK, ra0, rb0);
        else load_slice<T, VEC, GMN, false>(g, s, m0, n0, 0, ra0, rb0);
        store_slice<T>(smem, tid, ra0, rb0);
        if (nk > 1) load_slice<T, VEC, GMN, false>(g, s, m0, n0, k0_of(1), ra1, rb1);
        __syncthreads();
        int t = 0;
        constexpr int PARTS = T::A_VECS + T::B_VECS;
        constexpr int PER = (PARTS + T::HALF / 4 - 1) / (T::HALF / 4);   // groups per chunk
        // The loads are unconditional: past the end they re-read the last slice
        // (never stored), so the wait counts stay exact on every path.
        for (; t + 1 < nk; t += 2) {
            const int k2 = k0_of(t + 2 < nk ? t + 2 : nk - 1);
            const SliceRsrc r2 = slice_rsrc<T>(g, m0, n0, k2);
            compute_slice<T>(smem, wm, wn, lane, acc, [&](int c) {
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (c * PER + j < PARTS)
                        load_part<T, VEC, GMN, false>(g, s, m0, n0, k2, r2, c * PER + j, ra0, rb0);
            });
            store_slice<T>(smem + T::STAGE, tid, ra1, rb1);
            __syncthreads();
            const int k3 = k0_of(t + 3 < nk ? t + 3 : nk - 1);
            const SliceRsrc r3 = slice_rsrc<T>(g, m0, n0, k3);
            compute_slice<T>(smem + T::STAGE, wm, wn, lane, acc, [&](int c) {
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (c * PER + j < PARTS)
                        load_part<T, VEC, GMN, false>(g, s, m0, n0, k3, r3, c * PER + j, ra1, rb1);
            });
            if (t + 2 < nk) store_slice<T>(smem, tid, ra0, rb0);
            __syncthreads();
        }
        if (t < nk) compute_slice<T>(smem, wm, wn, lane, acc);
    }
}

// At least two waves per SIMD: with one wave per SIMD the matrix core idles
// whenever that wave waits at a barrier or on memory.
template <class T, bool VEC>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(2))) void sgemm_mfma_kernel(
    GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    f32x16 acc[T::MB][T::NB];
#pragma unroll
    for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
        for (int jb = 0; jb < T::NB; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ib][jb][r] = 0.f;

    const bool edge_mn = (m0 + T::BM > g.M) || (n0 + T::BN > g.N);
    if (edge_mn) k_loop<T, VEC, true>(g, m0, n0, tid, wm, wn, lane, smem, acc);
    else k_loop<T, VEC, false>(g, m0, n0, tid, wm, wn, lane, smem, acc);

    // Epilogue.  Accumulator register r of a 32x32 block holds, in lane l,
    // row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the block.  C is read in
    // a pass of its own before the first store: with a store between two C
    // loads the second load would have to wait for the first (the compiler
    // cannot tell their addresses apart), one memory round trip per element.
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const float alpha = g.alpha, beta = g.beta;
    float cv[T::MB][T::NB][16];
    if (beta != 0.f) {
#pragma unroll
        for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
            for (int jb = 0; jb < T::NB; ++jb) {
                const int col = n0 + wn * T::WN + jb * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * T::WM + ib * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool ok = !edge_mn || (row < g.M && col < g.N);
                    cv[ib][jb][r] = ok ? g.C[(int64_t)row * g.ldc + col] : 0.f;
                }
            }
    }
#pragma unroll
    for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
        for (int jb = 0; jb < T::NB; ++jb) {
            const int col = n0 + wn * T::WN + jb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * T::WM + ib * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (edge_mn && (row >= g.M || col >= g.N)) continue;
                float v = alpha * acc[ib][jb][r];
                if (beta != 0.f) v = fmaf(beta, cv[ib][jb][r], v);
                g.C[(int64_t)row * g.ldc + col] = v;
            }
        }
}

// 128x128 tiles: two slices in flight with 16-byte loads; one with 4-byte
// loads (whose staging registers would not fit two sets at two waves per SIMD).
using LargeTile = MfmaTile<128, 128, 32, 64, 64, 2>;
using LargeTileScalar = MfmaTile<128, 128, 32, 64, 64, 1>;
using SmallTile = MfmaTile<64, 64, 32, 32, 32>;

template <class TV, class TS>
hipError_t launch_tile(const GemmArgs &g, bool vec, int group_m, hipStream_t stream) {
    static_assert(TV::BM == TS::BM && TV::BN == TS::BN, "same tile");
    const int tiles_m = (g.M + TV::BM - 1) / TV::BM;
    const int tiles_n = (g.N + TV::BN - 1) / TV::BN;
    const dim3 grid(tiles_m * tiles_n);
    if (vec) hipLaunchKernelGGL((sgemm_mfma_kernel<TV, true>), grid, dim3(TV::NT), 0, stream, g, tiles_m, tiles_n, group_m);
    else hipLaunchKernelGGL((sgemm_mfma_kernel<TS, false>), grid, dim3(TS::NT), 0, stream, g, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

}  // namespace

int64_t mfma_large_grid(int M, int N) {
    return (int64_t)((M + LargeTile::BM - 1) / LargeTile::BM) * ((N + LargeTile::BN - 1) / LargeTile::BN);
}
int64_t mfma_small_grid(int M, int N) {
    return (int64_t)((M + SmallTile::BM - 1) / SmallTile::BM) * ((N + SmallTile::BN - 1) / SmallTile::BN);
}

hipError_t launch_mfma_large(const GemmArgs &g, bool vec_loads, hipStream_t stream) {
    return launch_tile<LargeTile, LargeTileScalar>(g, vec_loads, 8, stream);
}

hipError_t launch_mfma_small(const GemmArgs &g, bool vec_loads, hipStream_t stream) {
    return launch_tile<SmallTile, SmallTile>(g, vec_loads, 8, stream);
}

}  // namespace sgemm
