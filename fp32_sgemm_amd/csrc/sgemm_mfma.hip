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
// Staging.  Global loads are 16-byte buffer loads (buffer_load_dwordx4) where
// the operands are 16-byte aligned with row strides that are multiples of 4,
// four-byte loads otherwise.  Two LDS buffers alternate between slices (the
// double buffering of "Writing a Fast Matmul in CUDA, Step by Step", section
// "Bank conflicts and double buffering"): while the MFMAs of slice t read one
// buffer, the loads of a later slice are issued into registers, spread over
// slice t's MFMAs, and the next slice is written to the other buffer after
// them, so one barrier per slice separates producers from consumers.  The
// 16-byte configurations keep two slices in registers (t+1 waiting for its
// buffer, t+2 in flight), the others one.  The MFMAs of each slice's last
// chunk of fragments are issued after that barrier, while the next slice's
// first LDS reads are in flight.
//
// LDS layouts.  A 32x32x2 MFMA takes, in lane l, A(l % 32, k) and B(k, l % 32)
// for one of two k values picked by l / 32.  Inside a slice the kernel assigns
// lane half h = l / 32 the k range [h*BK/2, (h+1)*BK/2), so a lane walks a
// contiguous run of k for a fixed row of A and column of B.  Each operand is
// kept in LDS in its memory layout: one that is contiguous along k (A as given,
// B given transposed) keeps rows of k with a stride of BK + 4 floats and is
// read with ds_read_b128, four k steps per read; one that is contiguous along M
// or N (B as given, A given transposed) keeps rows of M or N and is read with
// ds_read_b32, the second half of the slice's k rows shifted by 32 floats so
// the two half-waves read opposite halves of the bank space.  The four operand
// forms (A and B each as given or transposed) are four instances of the same
// kernel.
//
// Edges.  Tiles that cross the M or N edge and the last slice when K is not a
// multiple of BK load through a guarded path that writes zeros for elements
// outside the matrices (adding exact zeros changes no sum), and edge tiles mask
// their stores.  The choice between guarded and plain loads is uniform across
// the work-group, so no barrier sits under divergent control flow.
//
// Epilogue.  C = alpha * acc + beta * C, where C is read only when beta != 0.
#include <atomic>
#include <type_traits>

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
// 4-byte vector-memory buffer store: offsets at or past the extent are
// dropped without a write.
__device__ void raw_buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.store.f32");

// A lane offset past every resource extent used here (extents stay below
// 2^31 bytes): the load returns zero and touches no memory.
constexpr int kOutOfRange = (int)0x80000000u;

// Buffer resource over [base, base + bytes): raw (untyped) access with the
// 32-bit data format, so every lane's offset is checked against `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes, 0x00020000);
}

// Memory layouts of an operand.  Both operands reach the matrix core in the
// same form: lane l supplies element (x = l % 32 of a block, k) of its operand,
// where x runs along M for A and along N for B.  They differ only in which
// index is contiguous in memory:
//   kKMajor: element (x, k) at X[x * ld + k]  (A as given; B given transposed)
//   kXMajor: element (x, k) at X[k * ld + x]  (B as given; A given transposed)
enum Layout : int { kKMajor = 0, kXMajor = 1 };

// Geometry of one operand's slice (BX values of x by BK values of k) as staged
// by NT threads, and its LDS form.  A kKMajor slice keeps its memory rows (one
// per x) with a row stride of BK + 4 floats, so the 16-byte fragment reads of 16
// consecutive rows fall in distinct banks.  A kXMajor slice keeps its memory
// rows (one per k) with the second half of the k rows shifted by 32 floats, so
// the two half-waves, which read rows k and k + BK/2, hit opposite halves of
// the bank space.
template <int BX_, int BK_, int NT_, int L_>
struct PanelGeom {
    static constexpr int X = BX_, BK = BK_, NT = NT_, L = L_;
    static constexpr int VECS = X * BK / 4 / NT;                    // 4-float groups per thread
    static constexpr int PER_ROW = (L == kKMajor ? BK : X) / 4;     // groups per memory row
    static constexpr int HALF = BK / 2;
    static constexpr int ROW_S = BK + 4;                            // kKMajor LDS row stride
    static constexpr int SHIFT = 32;                                // kXMajor offset of rows >= HALF
    static constexpr int STAGE = L == kKMajor ? X * ROW_S : BK * X + SHIFT;
    static_assert((X * BK) % (4 * NT) == 0, "load split");
};

template <int BM_, int BN_, int BK_, int WM_, int WN_, int PF_, int LA_, int LB_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int PF = PF_;             // slices loaded ahead of the one being computed
    // Two slices in flight: whether the next slice's LDS stores are spread over
    // this slice's chunks (one group after each chunk's loads) instead of
    // issued together after its MFMAs.  Taken for the 64x64 tiles, which run
    // one work-group per CU on the grids they serve: with one wave per SIMD,
    // in-order issue leaves the matrix core idle while a burst of stores goes
    // out.  Same-box per-launch medians (TFLOP/s): 1024^3 80.4 -> 85.6,
    // 1536^3 94.5 -> 99.0, 2048^3 131 -> 135.6, 512 x 512 x 8192 (8 splits)
    // 102.3 -> 105.9; the 128x128 tile on 6144 x 6144 x 2048 lost 1 %.
    static constexpr bool SPREAD = BM_ * BN_ <= 64 * 64;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = (BM / WM) * WAVES_N * 64;
    static constexpr int MB = WM / 32;          // 32x32 accumulator blocks per wave, along M
    static constexpr int NB = WN / 32;          // ... along N
    static constexpr int HALF = BK / 2;         // k values per lane half in one slice
    using PA = PanelGeom<BM, BK, NT, LA_>;
    using PB = PanelGeom<BN, BK, NT, LB_>;
    static constexpr int A_VECS = PA::VECS, B_VECS = PB::VECS;
    static constexpr int A_STAGE = PA::STAGE, B_STAGE = PB::STAGE;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    // Epilogue through LDS (interior tiles): the accumulators are written
    // row by row with a row stride of BN + 8 floats (rows four apart, which the
    // two half-waves write together, fall in opposite halves of the bank
    // space) and read back as 4-float groups, EPI_PARTS per thread,
    // consecutive threads along a row.
    static constexpr int EPI_S = BN + 8;
    static constexpr int EPI_PARTS = BM * BN / 4 / NT;
    static constexpr int EPI = BN >= 128 ? BM * EPI_S : 0;
    static constexpr int SMEM = 2 * STAGE > EPI ? 2 * STAGE : EPI;
    static_assert(SMEM * 4 <= 160 * 1024, "LDS");
    static_assert((BM * BN / 4) % NT == 0 && NT % (BN / 4) == 0, "epilogue groups");
};

// Per-thread addressing of the 4-float groups a thread stages from one operand
// for every slice: group i is memory row r[i], columns c[i]..c[i]+3 of the
// slice.  The row pointers (guarded loads) and the byte offsets from the slice
// origin (buffer loads of interior slices) are formed once.
template <class P>
struct Panel {
    const float *p[P::VECS];
    int r[P::VECS], c[P::VECS];
    int o[P::VECS];

    __device__ __forceinline__ Panel(const float *X, int64_t ld, int x0, int tid) {
#pragma unroll
        for (int i = 0; i < P::VECS; ++i) {
            const int q = tid + i * P::NT;
            r[i] = q / P::PER_ROW;
            c[i] = (q % P::PER_ROW) * 4;
            p[i] = P::L == kKMajor ? X + (int64_t)(x0 + r[i]) * ld + c[i] : X + (int64_t)r[i] * ld + x0 + c[i];
            o[i] = (r[i] * (int)ld + c[i]) * 4;
        }
    }
};

template <class T>
struct Stager {
    Panel<typename T::PA> a;
    Panel<typename T::PB> b;
    __device__ __forceinline__ Stager(const GemmArgs &g, int m0, int n0, int tid)
        : a(g.A, g.lda, m0, tid), b(g.B, g.ldb, n0, tid) {}
};

template <bool VEC>
__device__ __forceinline__ float4 ld4(const float *p) {
    if (VEC) return *reinterpret_cast<const float4 *>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}

// Resource over the elements of an operand's slice at k0 that lie inside the
// matrix: up to the last valid x (xn is the operand's extent along x).  For a
// kKMajor slice, rows past xn lie beyond the extent and read as zeros by
// themselves; in a kXMajor slice, columns past xn need an out-of-range lane
// offset (panel_load).
template <class P>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel_rsrc(const float *X, int64_t ld, int x0, int xn, int k0) {
    const int xs = min(P::X, xn - x0);
    if (P::L == kKMajor) return make_rsrc(X + (int64_t)x0 * ld + k0, (int)(((xs - 1) * ld + P::BK) * 4));
    return make_rsrc(X + (int64_t)k0 * ld + x0, (int)(((P::BK - 1) * ld + xs) * 4));
}

struct SliceRsrc {
    __amdgpu_buffer_rsrc_t a, b;
};

template <class T>
__device__ __forceinline__ SliceRsrc slice_rsrc(const GemmArgs &g, int m0, int n0, int k0) {
    SliceRsrc r;
    r.a = panel_rsrc<typename T::PA>(g.A, g.lda, m0, g.M, k0);
    r.b = panel_rsrc<typename T::PB>(g.B, g.ldb, n0, g.N, k0);
    return r;
}

// Loads 4-float group i of an operand's slice starting at k0.  GX: the tile
// crosses the M or N edge, so x >= xn reads as zero.  GK: the slice crosses the
// K edge, so k >= K reads as zero.  Nothing outside the matrix is accessed.
// Slices that do not cross the K edge are loaded with 16-byte buffer loads when
// VEC; the K-edge slice and 4-byte loads go through row pointers.
template <class P, bool VEC, bool GX, bool GK>
__device__ __forceinline__ float4 panel_load(const Panel<P> &s, __amdgpu_buffer_rsrc_t rs, int i, int64_t ld,
                                             int x0, int xn, int K, int k0) {
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr bool BUF = VEC && !GK;
    if (P::L == kKMajor) {
        const float *ptr = s.p[i] + k0;
        const bool row_ok = !GX || (x0 + s.r[i] < xn);
        if (BUF) {
            const f32x4v v = raw_buffer_load_v4f32(rs, s.o[i], 0, 0);
            return make_float4(v[0], v[1], v[2], v[3]);
        }
        if (!GK) return row_ok ? ld4<VEC>(ptr) : zero;
        const int k = k0 + s.c[i];
        float4 v = zero;
        if (row_ok) {
            if (k + 0 < K) v.x = ptr[0];
            if (k + 1 < K) v.y = ptr[1];
            if (k + 2 < K) v.z = ptr[2];
            if (k + 3 < K) v.w = ptr[3];
        }
        return v;
    } else {
        const float *ptr = s.p[i] + (int64_t)k0 * ld;
        const bool row_ok = !GK || (k0 + s.r[i] < K);
        if (BUF) {
            const int x = x0 + s.c[i];
            const int off = (!GX || x + 3 < xn) ? s.o[i] : kOutOfRange;
            const f32x4v v = raw_buffer_load_v4f32(rs, off, 0, 0);
            float4 w = make_float4(v[0], v[1], v[2], v[3]);
            if (GX && x < xn && x + 3 >= xn) {
                // The group straddles the edge (only when xn is not a multiple of 4).
                w.x = raw_buffer_load_f32(rs, s.o[i], 0, 0);
                w.y = raw_buffer_load_f32(rs, x + 1 < xn ? s.o[i] + 4 : kOutOfRange, 0, 0);
                w.z = raw_buffer_load_f32(rs, x + 2 < xn ? s.o[i] + 8 : kOutOfRange, 0, 0);
                w.w = 0.f;
            }
            return w;
        }
        if (!GX) return row_ok ? ld4<VEC>(ptr) : zero;
        const int x = x0 + s.c[i];
        float4 v = zero;
        if (row_ok) {
            if (VEC && x + 3 < xn) {
                v = ld4<true>(ptr);
            } else {
                if (x + 0 < xn) v.x = ptr[0];
                if (x + 1 < xn) v.y = ptr[1];
                if (x + 2 < xn) v.z = ptr[2];
                if (x + 3 < xn) v.w = ptr[3];
            }
        }
        return v;
    }
}

// Loads 4-float group p of the slice at k0: groups 0 .. A_VECS-1 are A's, the
// rest B's.  GMN: the tile crosses the M or N edge.
template <class T, bool VEC, bool GMN, bool GK>
__device__ __forceinline__ void load_part(const GemmArgs &g, const Stager<T> &s, int m0, int n0, int k0,
                                          const SliceRsrc &r, int p, float4 (&ra)[T::A_VECS],
                                          float4 (&rb)[T::B_VECS]) {
    if (p < T::A_VECS)
        ra[p] = panel_load<typename T::PA, VEC, GMN, GK>(s.a, r.a, p, g.lda, m0, g.M, g.K, k0);
    else
        rb[p - T::A_VECS] = panel_load<typename T::PB, VEC, GMN, GK>(s.b, r.b, p - T::A_VECS, g.ldb, n0, g.N, g.K, k0);
}

template <class T, bool VEC, bool GMN, bool GK>
__device__ __forceinline__ void load_slice(const GemmArgs &g, const Stager<T> &s, int m0, int n0, int k0,
                                           float4 (&ra)[T::A_VECS], float4 (&rb)[T::B_VECS]) {
    const SliceRsrc r = slice_rsrc<T>(g, m0, n0, k0);
#pragma unroll
    for (int p = 0; p < T::A_VECS + T::B_VECS; ++p) load_part<T, VEC, GMN, GK>(g, s, m0, n0, k0, r, p, ra, rb);
}

template <class P>
__device__ __forceinline__ void panel_store(float *S, int tid, const float4 (&v)[P::VECS]) {
#pragma unroll
    for (int i = 0; i < P::VECS; ++i) {
        const int q = tid + i * P::NT;
        const int r = q / P::PER_ROW, c = (q % P::PER_ROW) * 4;
        float *dst = P::L == kKMajor ? S + r * P::ROW_S + c : S + r * P::X + (r >= P::HALF ? P::SHIFT : 0) + c;
        *reinterpret_cast<float4 *>(dst) = v[i];
    }
}

template <class P>
__device__ __forceinline__ void panel_store_one(float *S, int tid, int i, const float4 &v) {
    const int q = tid + i * P::NT;
    const int r = q / P::PER_ROW, c = (q % P::PER_ROW) * 4;
    float *dst = P::L == kKMajor ? S + r * P::ROW_S + c : S + r * P::X + (r >= P::HALF ? P::SHIFT : 0) + c;
    *reinterpret_cast<float4 *>(dst) = v;
}

template <class T>
__device__ __forceinline__ void store_part(float *stage, int tid, int p, const float4 (&ra)[T::A_VECS],
                                           const float4 (&rb)[T::B_VECS]) {
    if (p < T::A_VECS) panel_store_one<typename T::PA>(stage, tid, p, ra[p]);
    else panel_store_one<typename T::PB>(stage + T::A_STAGE, tid, p - T::A_VECS, rb[p - T::A_VECS]);
}

template <class T>
__device__ __forceinline__ void store_slice(float *stage, int tid, const float4 (&ra)[T::A_VECS],
                                            const float4 (&rb)[T::B_VECS]) {
    panel_store<typename T::PA>(stage, tid, ra);
    panel_store<typename T::PB>(stage + T::A_STAGE, tid, rb);
}

// LDS address of a lane's first fragment element in an operand's stage: x =
// xw + l % 32 (xw is the wave's offset along x) and k = h * BK/2, h = l / 32.
template <class P>
__device__ __forceinline__ const float *panel_lane(const float *S, int xw, int l32, int h) {
    if (P::L == kKMajor) return S + (xw + l32) * P::ROW_S + h * P::HALF;
    return S + h * (P::HALF * P::X + P::SHIFT) + xw + l32;
}

// Chunk c (4 k steps) of a lane's fragments for NBLK 32-wide blocks along x:
// f[b][e] is the element at x + 32 b and k + 4 c + e.  A kKMajor stage gives the
// four k in one 16-byte read, a kXMajor stage one float per k.
template <class P, int NBLK>
__device__ __forceinline__ void panel_frag(const float *base, int c, float (&f)[NBLK][4]) {
    if (P::L == kKMajor) {
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const float4 v = *reinterpret_cast<const float4 *>(base + b * 32 * P::ROW_S + 4 * c);
            f[b][0] = v.x;
            f[b][1] = v.y;
            f[b][2] = v.z;
            f[b][3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int b = 0; b < NBLK; ++b) f[b][e] = base[(4 * c + e) * P::X + b * 32];
    }
}

// Fragments of one chunk of a slice for all of the wave's blocks.
template <class T>
struct Frag {
    float a[T::MB][4];
    float b[T::NB][4];
};

template <class T>
__device__ __forceinline__ void read_frag(const float *As, const float *Bs, int c, Frag<T> &f) {
    panel_frag<typename T::PA, T::MB>(As, c, f.a);
    panel_frag<typename T::PB, T::NB>(Bs, c, f.b);
}

template <class T>
__device__ __forceinline__ void mfma_frag(const Frag<T> &f, f32x16 (&acc)[T::MB][T::NB]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
            for (int jb = 0; jb < T::NB; ++jb)
                acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[ib][e], f.b[jb][e], acc[ib][jb], 0, 0, 0);
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
    const float *As = panel_lane<typename T::PA>(stage, wm * T::WM, l32, h);
    const float *Bs = panel_lane<typename T::PB>(stage + T::A_STAGE, wn * T::WN, l32, h);
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

// As compute_slice, with the MFMAs of each slice's last chunk held back: on
// entry f[1] holds the previous slice's last chunk (zeros before the first
// slice), whose MFMAs run right after this slice's first LDS reads are issued,
// so that the matrix cores stay busy while those reads are in flight (after
// the barrier that precedes every slice); on return f[1] holds this slice's
// last chunk, not yet multiplied.  The caller runs it after the last slice.
template <class T, class Issue>
__device__ __forceinline__ void compute_slice_held(const float *stage, int wm, int wn, int lane,
                                                   f32x16 (&acc)[T::MB][T::NB], const Issue &issue,
                                                   Frag<T> (&f)[2]) {
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const float *As = panel_lane<typename T::PA>(stage, wm * T::WM, l32, h);
    const float *Bs = panel_lane<typename T::PB>(stage + T::A_STAGE, wn * T::WN, l32, h);
    constexpr int CH = T::HALF / 4;
    static_assert(CH % 2 == 0, "held chunk must land in f[1]");
    read_frag<T>(As, Bs, 0, f[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_frag<T>(f[1], acc);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        issue(c);
        if (c + 1 < CH) {
            read_frag<T>(As, Bs, c + 1, f[(c + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag<T>(f[c & 1], acc);
        }
    }
}

template <class T>
__device__ __forceinline__ void zero_frag(Frag<T> &f) {
#pragma unroll
    for (int b = 0; b < T::MB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) f.a[b][e] = 0.f;
#pragma unroll
    for (int b = 0; b < T::NB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) f.b[b][e] = 0.f;
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
        // One register set: slice t+1 is loaded during slice t's MFMAs and
        // stored into the other LDS stage after them.
        float4 ra[T::A_VECS], rb[T::B_VECS];
        if (tail) load_slice<T, VEC, GMN, true>(g, s, m0, n0, nkf * T::BK, ra, rb);
        else load_slice<T, VEC, GMN, false>(g, s, m0, n0, 0, ra, rb);
        store_slice<T>(smem, tid, ra, rb);
        __syncthreads();
        if (nk == 1) {
            compute_slice<T>(smem, wm, wn, lane, acc);
            return;
        }
        constexpr int PARTS = T::A_VECS + T::B_VECS;
        constexpr int PER = (PARTS + T::HALF / 4 - 1) / (T::HALF / 4);   // groups per chunk
        Frag<T> f[2];
        zero_frag<T>(f[1]);
        for (int t = 0; t < nk; ++t) {
            // Past the end the last slice is loaded again and never stored.
            const int k1 = k0_of(t + 1 < nk ? t + 1 : nk - 1);
            const SliceRsrc r1 = slice_rsrc<T>(g, m0, n0, k1);
            compute_slice_held<T>(smem + (t & 1) * T::STAGE, wm, wn, lane, acc, [&](int c) {
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (c * PER + j < PARTS) load_part<T, VEC, GMN, false>(g, s, m0, n0, k1, r1, c * PER + j, ra, rb);
            }, f);
            if (t + 1 < nk) store_slice<T>(smem + ((t + 1) & 1) * T::STAGE, tid, ra, rb);
            __syncthreads();
        }
        mfma_frag<T>(f[1], acc);
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
        Frag<T> f[2];
        zero_frag<T>(f[1]);
        // The loads are unconditional: past the end they re-read the last slice
        // (never stored), so the wait counts stay exact on every path.
        for (; t + 1 < nk; t += 2) {
            const int k2 = k0_of(t + 2 < nk ? t + 2 : nk - 1);
            const SliceRsrc r2 = slice_rsrc<T>(g, m0, n0, k2);
            compute_slice_held<T>(smem, wm, wn, lane, acc, [&](int c) {
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (c * PER + j < PARTS) {
                        if (T::SPREAD) store_part<T>(smem + T::STAGE, tid, c * PER + j, ra1, rb1);
                        load_part<T, VEC, GMN, false>(g, s, m0, n0, k2, r2, c * PER + j, ra0, rb0);
                    }
            }, f);
            if (!T::SPREAD) store_slice<T>(smem + T::STAGE, tid, ra1, rb1);
            __syncthreads();
            const int k3 = k0_of(t + 3 < nk ? t + 3 : nk - 1);
            const SliceRsrc r3 = slice_rsrc<T>(g, m0, n0, k3);
            const bool st0 = t + 2 < nk;
            compute_slice_held<T>(smem + T::STAGE, wm, wn, lane, acc, [&](int c) {
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (c * PER + j < PARTS) {
                        if (T::SPREAD && st0) store_part<T>(smem, tid, c * PER + j, ra0, rb0);
                        load_part<T, VEC, GMN, false>(g, s, m0, n0, k3, r3, c * PER + j, ra1, rb1);
                    }
            }, f);
            if (!T::SPREAD && st0) store_slice<T>(smem, tid, ra0, rb0);
            __syncthreads();
        }
        if (t < nk) compute_slice_held<T>(smem, wm, wn, lane, acc, NoIssue(), f);
        mfma_frag<T>(f[1], acc);
    }
}

// Split of the reduction over work-groups (split-K, "Writing a Fast Matmul in
// CUDA, Step by Step", section "In the real world": too few output tiles to
// fill the GPU, so the K loop is divided and the partial results added).  Split
// s of `splits` covers k in [s*k_per, min(K, (s+1)*k_per)), k_per a multiple of
// BK, and writes its unscaled partial product to ws + s*M*N (row-major, row
// stride N); splitk_reduce_kernel then adds the partials in split order.
struct SplitK {
    int splits;
    int k_per;
    float *ws;
};

// Operands moved to the K range [kb, kb + klen) of the product.
template <class T>
__device__ __forceinline__ void shift_k(GemmArgs &g, int kb, int klen) {
    g.A += T::PA::L == kKMajor ? (int64_t)kb : (int64_t)kb * g.lda;
    g.B += T::PB::L == kXMajor ? (int64_t)kb * g.ldb : (int64_t)kb;
    g.K = klen;
}

// One output tile at (m0, n0) over g's K range: Cb = alpha * acc + beta * Cb,
// where Cb points at the tile's first element with row stride ldc (C itself,
// or a partial-sum slot).  Elements outside M x N are neither read nor
// written.
template <class T, bool VEC, bool LDS_EPI = true>
__device__ __forceinline__ void compute_tile(const GemmArgs &g, int m0, int n0, float *smem, float *Cb,
                                             int64_t ldc, float alpha, float beta) {
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

    // Interior tiles 128 wide of a 16-byte aligned C whose row stride is a
    // multiple of 4 (and whose tile spans less than 2 GiB) go through LDS, so
    // C is read and written in 4-float groups along its rows: 512-byte row
    // segments per half-wave instead of 128-byte ones (64-wide tiles gained
    // nothing).  Not in the persistent kernel, whose registers it would crowd.
    if (LDS_EPI && T::BN >= 128 && !edge_mn && (reinterpret_cast<uintptr_t>(Cb) % 16 == 0) && (ldc % 4 == 0) &&
        (int64_t)(T::BM - 1) * ldc * 4 + T::BN * 4 < ((int64_t)1 << 31)) {
        constexpr int GPR = T::BN / 4;            // 4-float groups per tile row
        constexpr int GROWS = T::NT / GPR;        // tile rows per group index
        const int grow = tid / GPR, gcol = 4 * (tid % GPR);
        const int h = lane >> 5, l32 = lane & 31;
        // C's groups are requested first, so their latency overlaps the
        // accumulators' trip through LDS.
        float4 cv[T::EPI_PARTS];
        if (beta != 0.f) {
#pragma unroll
            for (int p = 0; p < T::EPI_PARTS; ++p)
                cv[p] = *reinterpret_cast<const float4 *>(Cb + (int64_t)(p * GROWS + grow) * ldc + gcol);
        }
        __syncthreads();   // every wave is done reading the LDS stages
#pragma unroll
        for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
            for (int jb = 0; jb < T::NB; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = wm * T::WM + ib * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    smem[rr * T::EPI_S + wn * T::WN + jb * 32 + l32] = acc[ib][jb][r];
                }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < T::EPI_PARTS; ++p) {
            const float4 a = *reinterpret_cast<const float4 *>(smem + (p * GROWS + grow) * T::EPI_S + gcol);
            float4 v = make_float4(alpha * a.x, alpha * a.y, alpha * a.z, alpha * a.w);
            if (beta != 0.f) {
                v.x = fmaf(beta, cv[p].x, v.x);
                v.y = fmaf(beta, cv[p].y, v.y);
                v.z = fmaf(beta, cv[p].z, v.z);
                v.w = fmaf(beta, cv[p].w, v.w);
            }
            // C is written once and not read again here: a non-temporal
            // store keeps it from displacing the A and B panels in L2.
            const f32x4v w = {v.x, v.y, v.z, v.w};
            __builtin_nontemporal_store(w, reinterpret_cast<f32x4v *>(Cb + (int64_t)(p * GROWS + grow) * ldc + gcol));
        }
        return;
    }

    // Epilogue.  Accumulator register r of a 32x32 block holds, in lane l,
    // row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the block.  C is read in
    // a pass of its own before the first store: with a store between two C
    // loads the second load would have to wait for the first (the compiler
    // cannot tell their addresses apart), one memory round trip per element.
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int rows = g.M - m0, cols = g.N - n0;
    // Interior tiles take a copy of the epilogue without any per-element
    // guard: straight-line code lets the compiler wait for each C load only
    // as far as needed, instead of for all outstanding loads at every guarded
    // element.  Edge tiles keep it branch-free too, through a buffer resource
    // over the tile's valid part of C: rows past M lie beyond its extent and
    // columns past N get an out-of-range offset, so their loads read zero and
    // their stores are dropped.  (When 128 rows of C span 2 GiB or more, edge
    // tiles fall back to guarded pointer accesses.)
    const bool buf_edge = (int64_t)(T::BM - 1) * ldc * 4 + T::BN * 4 < ((int64_t)1 << 31);
    auto epilogue = [&](auto mode_tag) {
        constexpr int MODE = decltype(mode_tag)::value;   // 0 interior, 1 edge via buffer, 2 edge guarded
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(Cb, MODE == 1 ? (int)(((int64_t)(min(rows, T::BM) - 1) * ldc + min(cols, T::BN)) * 4) : 0);
        float cv[T::MB][T::NB][16];
        if (beta != 0.f) {
#pragma unroll
            for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
                for (int jb = 0; jb < T::NB; ++jb) {
                    const int c = wn * T::WN + jb * 32 + l32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rr = wm * T::WM + ib * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (MODE == 0) {
                            cv[ib][jb][r] = Cb[(int64_t)rr * ldc + c];
                        } else if (MODE == 1) {
                            cv[ib][jb][r] = raw_buffer_load_f32(rc, c < cols ? (int)((rr * ldc + c) * 4) : kOutOfRange, 0, 0);
                        } else {
                            const bool ok = rr < rows && c < cols;
                            cv[ib][jb][r] = ok ? Cb[(int64_t)rr * ldc + c] : 0.f;
                        }
                    }
                }
        }
#pragma unroll
        for (int ib = 0; ib < T::MB; ++ib)
#pragma unroll
            for (int jb = 0; jb < T::NB; ++jb) {
                const int c = wn * T::WN + jb * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = wm * T::WM + ib * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    float v = alpha * acc[ib][jb][r];
                    if (beta != 0.f) v = fmaf(beta, cv[ib][jb][r], v);
                    if (MODE == 0) {
                        Cb[(int64_t)rr * ldc + c] = v;
                    } else if (MODE == 1) {
                        raw_buffer_store_f32(v, rc, c < cols ? (int)((rr * ldc + c) * 4) : kOutOfRange, 0, 0);
                    } else if (rr < rows && c < cols) {
                        Cb[(int64_t)rr * ldc + c] = v;
                    }
                }
            }
    };
    if (!edge_mn) epilogue(std::integral_constant<int, 0>());
    else if (buf_edge) epilogue(std::integral_constant<int, 1>());
    else epilogue(std::integral_constant<int, 2>());
}

// At least two waves per SIMD: with one wave per SIMD the matrix core idles
// whenever that wave waits at a barrier or on memory.
// `ntiles`: the launch covers tiles [0, ntiles) of the grouped tile order (all
// of them, or the whole rounds ahead of a stream-K part).
template <class T, bool VEC>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(2))) void sgemm_mfma_kernel(
    GemmArgs g, int tiles_m, int tiles_n, int group_m, int ntiles, SplitK sk) {
    __shared__ __attribute__((aligned(16))) float smem[T::SMEM];
    poison_lds<sizeof(smem)>(smem);

    int bid = blockIdx.x;
    float *Cbase = g.C;
    int64_t ldc = g.ldc;
    float alpha = g.alpha, beta = g.beta;
    if (sk.splits > 1) {
        // Work-groups [s*ntiles, (s+1)*ntiles) compute split s: the same
        // product on a K range, written unscaled to the split's partial slab.
        const int sp = bid / ntiles;
        bid -= sp * ntiles;
        const int kb = sp * sk.k_per;
        shift_k<T>(g, kb, min(sk.k_per, g.K - kb));
        Cbase = sk.ws + (int64_t)sp * g.M * g.N;
        ldc = g.N;
        alpha = 1.f;
        beta = 0.f;
    }
    int tm, tn;
    tile_coords(xcd_position(bid, ntiles), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    compute_tile<T, VEC>(g, m0, n0, smem, Cbase + (int64_t)m0 * ldc + n0, ldc, alpha, beta);
}

// ---------------------------------------------------------------------------
// Persistent, tile-scheduled form (data-parallel rounds plus stream-K).
//
// With T tiles and P resident work-groups, whole rounds of P tiles leave a
// last round only partly filled ("Writing a Fast Matmul in CUDA, Step by
// Step", section "Size effects": a second wave that runs a third full).  A
// persistent kernel keeps its work-groups alive across several output tiles
// ("CUDA Matrix Multiplication Optimization: From Naive to Near-cuBLAS",
// section "Beyond Tiling: Async, Tensor Cores, and Scheduling").  Here
// Whole rounds of P tiles run first as an ordinary grid (floor(T/P) rounds,
// one fewer when T/P leaves a remainder).  Then P work-groups stay resident
// and each takes an equal share of the remaining tiles' K slices ("units", ipt
// per tile), a contiguous range that may begin or end inside a tile.  A tile computed whole writes C; a piece of a tile writes its
// unscaled partial sum to one of two slots of its work-group (slot 0: the
// piece that starts the work-group's range inside a tile begun by an earlier
// work-group; slot 1: the piece that ends the range inside a tile continued by
// a later one), and streamk_fixup_kernel adds each split tile's pieces in K
// order.  No work-group ever waits for another.
// ---------------------------------------------------------------------------
struct StreamK {
    int P;              // resident work-groups (a multiple of 8)
    int rounds;         // whole-tile rounds (run by the grid kernel first)
    int ipt;            // K slices per tile
    int rem_begin;      // first tile of the stream-K part
    int64_t units;      // K slices of the stream-K part: (tiles - rounds*P) * ipt
    float *ws;          // 2 * P slots of BM*BN floats
};

// Work-group w's units of the stream-K part: [unit_begin(w), unit_begin(w+1)).
__host__ __device__ __forceinline__ int64_t unit_begin(const StreamK &sk, int w) {
    return (int64_t)w * sk.units / sk.P;
}
// The work-group whose range holds unit u.
__host__ __device__ __forceinline__ int owner_of_unit(const StreamK &sk, int64_t u) {
    return (int)(((u + 1) * sk.P - 1) / sk.units);
}

template <class T, bool VEC>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(2))) void sgemm_mfma_streamk_kernel(
    GemmArgs g, int tiles_m, int tiles_n, int group_m, StreamK sk) {
    __shared__ __attribute__((aligned(16))) float smem[T::SMEM];
    poison_lds<sizeof(smem)>(smem);
    // Work-groups resident on one XCD take consecutive positions, so they
    // work on neighbouring tiles and share their panels in that XCD's L2.
    const int w = xcd_position(blockIdx.x, sk.P);
    const int64_t u1 = unit_begin(sk, w + 1);
    for (int64_t u = unit_begin(sk, w); u < u1;) {
        const int rt = (int)(u / sk.ipt);
        const int j0 = (int)(u - (int64_t)rt * sk.ipt);
        const int j1 = (int)min((int64_t)sk.ipt, j0 + (u1 - u));
        const int t = sk.rem_begin + rt;
        u += j1 - j0;
        int tm, tn;
        tile_coords(t, tiles_m, tiles_n, group_m, tm, tn);
        const int m0 = tm * T::BM, n0 = tn * T::BN;
        GemmArgs gs = g;
        const int kb = j0 * T::BK;
        shift_k<T>(gs, kb, min(g.K, j1 * T::BK) - kb);
        const bool whole = j0 == 0 && j1 == sk.ipt;
        float *Cb = whole ? g.C + (int64_t)m0 * g.ldc + n0
                          : sk.ws + (int64_t)(2 * w + (j0 > 0 ? 0 : 1)) * (T::BM * T::BN);
        compute_tile<T, VEC, false>(gs, m0, n0, smem, Cb, whole ? g.ldc : (int64_t)T::BN,
                                    whole ? g.alpha : 1.f, whole ? g.beta : 0.f);
        __syncthreads();
    }
}

// One work-group per boundary between work-groups w-1 and w of the stream-K
// part that falls inside a tile; only the first such boundary of a tile does
// the work: C = alpha * (pieces in K order) + beta * C over the tile.
template <int BM, int BN>
__global__ __launch_bounds__(256) void streamk_fixup_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m,
                                                            StreamK sk) {
    const int w = blockIdx.x + 1;
    const int64_t b = unit_begin(sk, w);
    if (b >= sk.units || b % sk.ipt == 0) return;
    const int64_t first = b / sk.ipt * sk.ipt;
    if (unit_begin(sk, w - 1) > first) return;
    const int wf = w - 1;
    const int wl = owner_of_unit(sk, first + sk.ipt - 1);
    int tm, tn;
    tile_coords(sk.rem_begin + (int)(b / sk.ipt), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows = min(BM, g.M - m0), cols = min(BN, g.N - n0);
    constexpr int SLOT = BM * BN;
    static_assert(BN % 4 == 0, "groups of 4 columns");
    // Each thread adds groups of 4 columns (16-byte reads of the slots).
    for (int e = 4 * threadIdx.x; e < SLOT; e += 4 * 256) {
        const int r = e / BN, c = e % BN;
        if (r >= rows || c >= cols) continue;
        float4 s = *reinterpret_cast<const float4 *>(sk.ws + (int64_t)(2 * wf + 1) * SLOT + e);
        // Work-groups with an empty range (fewer units than work-groups) hold
        // no piece.
        for (int v = wf + 1; v <= wl; ++v) {
            if (unit_begin(sk, v) == unit_begin(sk, v + 1)) continue;
            const float4 x = *reinterpret_cast<const float4 *>(sk.ws + (int64_t)(2 * v) * SLOT + e);
            s.x += x.x;
            s.y += x.y;
            s.z += x.z;
            s.w += x.w;
        }
        const float sv[4] = {s.x, s.y, s.z, s.w};
        float *p = g.C + (int64_t)(m0 + r) * g.ldc + n0 + c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (c + q >= cols) break;
            float out = g.alpha * sv[q];
            if (g.beta != 0.f) out = fmaf(g.beta, p[q], out);
            p[q] = out;
        }
    }
}

// Sum of the partials ws[sp * total + t], sp = 0 .. splits-1, added in split
// order.  The loads go out eight at a time before their additions (with a
// run-time loop bound each addition would otherwise wait for its own load,
// one memory round trip per split); indices past the last split re-read it
// and are not added.
template <class V>
__device__ __forceinline__ V add_splits(const float *ws, int64_t total, int64_t t, int splits) {
    constexpr int B = 8;
    V sum = *reinterpret_cast<const V *>(ws + t);
    for (int sp0 = 1; sp0 < splits; sp0 += B) {
        V v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int sp = sp0 + j < splits ? sp0 + j : splits - 1;
            v[j] = *reinterpret_cast<const V *>(ws + sp * total + t);
        }
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (sp0 + j < splits) sum = sum + v[j];
    }
    return sum;
}

// C = alpha * (the split partials added in split order) + beta * C.  VEC4: N,
// ldc and C allow 16-byte accesses, so each thread takes four columns.
template <bool VEC4>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, const float *ws, int splits) {
    const int64_t total = (int64_t)g.M * g.N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float alpha = g.alpha, beta = g.beta;
    if (VEC4) {
        for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total / 4; q += stride) {
            const int64_t t = 4 * q;
            const float4 sum = add_splits<float4>(ws, total, t, splits);
            const int64_t i = t / g.N, j = t - i * g.N;
            float4 *p = reinterpret_cast<float4 *>(g.C + i * g.ldc + j);
            float4 r = make_float4(alpha * sum.x, alpha * sum.y, alpha * sum.z, alpha * sum.w);
            if (beta != 0.f) {
                const float4 c = *p;
                r = make_float4(fmaf(beta, c.x, r.x), fmaf(beta, c.y, r.y), fmaf(beta, c.z, r.z),
                                fmaf(beta, c.w, r.w));
            }
            *p = r;
        }
    } else {
        for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
            const float sum = add_splits<float>(ws, total, t, splits);
            const int64_t i = t / g.N, j = t - i * g.N;
            float *p = g.C + i * g.ldc + j;
            float v = alpha * sum;
            if (beta != 0.f) v = fmaf(beta, *p, v);
            *p = v;
        }
    }
}

// Tile configurations.  128x128: two slices in flight with 16-byte loads, one
// with 4-byte loads (whose staging registers would not fit two sets at two
// waves per SIMD).  The others are shapes for grids that 128x128 tiles would
// leave short of work-groups.
template <int LA, int LB>
using LargeTile = MfmaTile<128, 128, 32, 64, 64, 2, LA, LB>;
template <int LA, int LB>
using LargeTileScalar = MfmaTile<128, 128, 32, 64, 64, 1, LA, LB>;
template <int LA, int LB>
using SmallTile = MfmaTile<64, 64, 32, 32, 32, 1, LA, LB>;
template <int LA, int LB>
using TallTile = MfmaTile<128, 64, 32, 64, 32, 2, LA, LB>;
template <int LA, int LB>
using WideTile = MfmaTile<64, 128, 32, 32, 64, 2, LA, LB>;
template <int LA, int LB>
using SmallTile2 = MfmaTile<64, 64, 32, 32, 32, 2, LA, LB>;
// 64x64 with slices of 64: twice the MFMA work per slice, so the two slices in
// flight cover twice the memory latency (grids of at most one work-group per
// compute unit, where no other work-group hides it).
template <int LA, int LB>
using SmallTileK64 = MfmaTile<64, 64, 64, 32, 32, 2, LA, LB>;

constexpr int kTileBM[kNumMfmaConfigs] = {128, 64, 128, 64, 64, 128, 64, 256, 128, 64, 192};
constexpr int kTileBN[kNumMfmaConfigs] = {128, 64, 64, 128, 64, 128, 64, 256, 128, 64, 192};
constexpr int kTileBK = 32;

template <class T, bool VEC>
hipError_t launch_one(const GemmArgs &g, int group_m, const SplitK &sk, hipStream_t stream) {
    const int tiles_m = (g.M + T::BM - 1) / T::BM;
    const int tiles_n = (g.N + T::BN - 1) / T::BN;
    const dim3 grid(tiles_m * tiles_n * sk.splits);
    hipLaunchKernelGGL((sgemm_mfma_kernel<T, VEC>), grid, dim3(T::NT), 0, stream, g, tiles_m, tiles_n, group_m,
                       tiles_m * tiles_n, sk);
    return hipGetLastError();
}

// Work-groups of the persistent kernel that fit on the device at once (a
// multiple of 8, one share per XCD), cached per device.
template <class T>
hipError_t resident_groups(int *out) {
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
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sgemm_mfma_streamk_kernel<T, true>, T::NT, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int P = per_cu * cus / kNumXcd * kNumXcd;
    if (P < kNumXcd) P = kNumXcd;
    if (dev >= 0 && dev < 64) cache[dev].store(P, std::memory_order_relaxed);
    *out = P;
    return hipSuccess;
}

// The stream-K plan's split: whole rounds of P resident work-groups, then the
// remaining tiles' K slices in equal shares.  With a remainder, the last whole
// round joins the stream-K part, so each work-group's share is at least one
// tile's K slices and a tile is cut at most once ("data-parallel plus one-tile
// stream-K").
template <class T>
hipError_t streamk_plan(const GemmArgs &g, StreamK *sk, int *tiles_m, int *tiles_n) {
    *tiles_m = (g.M + T::BM - 1) / T::BM;
    *tiles_n = (g.N + T::BN - 1) / T::BN;
    const int tiles = *tiles_m * *tiles_n;
    hipError_t e = resident_groups<T>(&sk->P);
    if (e != hipSuccess) return e;
    sk->ipt = (g.K + T::BK - 1) / T::BK;
    sk->rounds = tiles / sk->P;
    if (sk->rounds > 0 && tiles % sk->P != 0) sk->rounds -= 1;
    sk->rem_begin = sk->rounds * sk->P;
    sk->units = (int64_t)(tiles - sk->rem_begin) * sk->ipt;
    sk->ws = nullptr;
    return hipSuccess;
}

template <class T>
int64_t streamk_scratch_bytes(const StreamK &sk) {
    return sk.units == 0 ? 0 : (int64_t)2 * sk.P * T::BM * T::BN * (int64_t)sizeof(float);
}

template <class T>
hipError_t launch_streamk(const GemmArgs &g, int group_m, hipStream_t stream) {
    StreamK sk;
    int tiles_m = 0, tiles_n = 0;
    hipError_t e = streamk_plan<T>(g, &sk, &tiles_m, &tiles_n);
    if (e != hipSuccess) return e;
    if (sk.units > 0) {
        e = scratch_acquire(g.scratch, (size_t)streamk_scratch_bytes<T>(sk), stream,
                            reinterpret_cast<void **>(&sk.ws));
        if (e != hipSuccess) return e;
    }
    // The whole rounds run as an ordinary grid over their tiles (the grid
    // kernel keeps fewer registers live than the persistent loop); the
    // persistent kernel takes the stream-K part only.
    if (sk.rounds > 0) {
        SplitK none{1, g.K, nullptr};
        hipLaunchKernelGGL((sgemm_mfma_kernel<T, true>), dim3(sk.rounds * sk.P), dim3(T::NT), 0, stream, g,
                           tiles_m, tiles_n, group_m, sk.rounds * sk.P, none);
        e = hipGetLastError();
    }
    if (sk.units > 0) {
        sk.rounds = 0;
        if (e == hipSuccess) {
            hipLaunchKernelGGL((sgemm_mfma_streamk_kernel<T, true>), dim3(sk.P), dim3(T::NT), 0, stream, g,
                               tiles_m, tiles_n, group_m, sk);
            e = hipGetLastError();
        }
        if (e == hipSuccess && sk.P >= 2) {
            hipLaunchKernelGGL((streamk_fixup_kernel<T::BM, T::BN>), dim3(sk.P - 1), dim3(256), 0, stream, g,
                               tiles_m, tiles_n, group_m, sk);
            e = hipGetLastError();
        }
        const hipError_t r = scratch_release(g.scratch, sk.ws, stream);
        if (e == hipSuccess) e = r;
    }
    return e;
}

template <int LA, int LB>
hipError_t launch_layouts(const GemmArgs &g, int config, bool vec, int group_m, const SplitK &sk,
                          hipStream_t stream) {
    switch (config) {
        case 0:
            return vec ? launch_one<LargeTile<LA, LB>, true>(g, group_m, sk, stream)
                       : launch_one<LargeTileScalar<LA, LB>, false>(g, group_m, sk, stream);
        case 1:
            return vec ? launch_one<SmallTile<LA, LB>, true>(g, group_m, sk, stream)
                       : launch_one<SmallTile<LA, LB>, false>(g, group_m, sk, stream);
        case 2: return launch_one<TallTile<LA, LB>, true>(g, group_m, sk, stream);
        case 3: return launch_one<WideTile<LA, LB>, true>(g, group_m, sk, stream);
        case 4: return launch_one<SmallTile2<LA, LB>, true>(g, group_m, sk, stream);
        case 5: return launch_streamk<LargeTile<LA, LB>>(g, group_m, stream);
        case 6: return launch_one<SmallTileK64<LA, LB>, true>(g, group_m, sk, stream);
        case 7: return launch_big(g, stream);
        case 8: return launch_dl128(g, group_m, stream);
        case 9: return launch_dl64(g, group_m, stream);
        case 10: return launch_dl192(g, group_m, stream);
        default: return hipErrorInvalidValue;
    }
}

// A as given is kKMajor and B kXMajor; a transposed operand swaps its layout.
hipError_t launch_kernel(const GemmArgs &g, int config, bool vec, int group_m, const SplitK &sk,
                         hipStream_t stream) {
    const bool ta = g.trans_a != 0, tb = g.trans_b != 0;
    if (!ta && !tb) return launch_layouts<kKMajor, kXMajor>(g, config, vec, group_m, sk, stream);
    if (!ta && tb) return launch_layouts<kKMajor, kKMajor>(g, config, vec, group_m, sk, stream);
    if (ta && !tb) return launch_layouts<kXMajor, kXMajor>(g, config, vec, group_m, sk, stream);
    return launch_layouts<kXMajor, kKMajor>(g, config, vec, group_m, sk, stream);
}

}  // namespace

int64_t mfma_config_tiles(int config, int M, int N) {
    if (config < 0 || config >= kNumMfmaConfigs) return -1;
    return (int64_t)((M + kTileBM[config] - 1) / kTileBM[config]) * ((N + kTileBN[config] - 1) / kTileBN[config]);
}
int64_t mfma_large_grid(int M, int N) { return mfma_config_tiles(0, M, N); }
int64_t mfma_small_grid(int M, int N) { return mfma_config_tiles(1, M, N); }

bool mfma_config_scalar_ok(int config) { return config == 0 || config == 1; }
bool mfma_config_splits_ok(int config) { return config != 5 && config < 7; }

int mfma_effective_splits(int K, int splits, int *k_per) {
    if (splits < 1) splits = 1;
    int per = (K + splits - 1) / splits;
    per = (per + kTileBK - 1) / kTileBK * kTileBK;
    if (per < kTileBK) per = kTileBK;
    *k_per = per;
    return (K + per - 1) / per;
}

namespace {

// Scratch of the stream-K plan for operand layouts LA, LB (its occupancy, and
// so its number of resident work-groups, follows the layouts' LDS use).
template <int LA, int LB>
hipError_t streamk_bytes(const GemmArgs &g, int64_t *bytes) {
    StreamK sk;
    int tiles_m = 0, tiles_n = 0;
    const hipError_t e = streamk_plan<LargeTile<LA, LB>>(g, &sk, &tiles_m, &tiles_n);
    if (e != hipSuccess) return e;
    *bytes = streamk_scratch_bytes<LargeTile<LA, LB>>(sk);
    return hipSuccess;
}

}  // namespace

hipError_t mfma_config_scratch_bytes(const GemmArgs &g, int config, int splits, int64_t *bytes) {
    *bytes = 0;
    if (config == 5) {
        const bool ta = g.trans_a != 0, tb = g.trans_b != 0;
        if (!ta && !tb) return streamk_bytes<kKMajor, kXMajor>(g, bytes);
        if (!ta && tb) return streamk_bytes<kKMajor, kKMajor>(g, bytes);
        if (ta && !tb) return streamk_bytes<kXMajor, kXMajor>(g, bytes);
        return streamk_bytes<kXMajor, kKMajor>(g, bytes);
    }
    if (!mfma_config_splits_ok(config)) return hipSuccess;
    int k_per = 0;
    const int eff = mfma_effective_splits(g.K, splits, &k_per);
    if (eff > 1) *bytes = (int64_t)eff * g.M * g.N * (int64_t)sizeof(float);
    return hipSuccess;
}

hipError_t launch_mfma_config(const GemmArgs &g, int config, bool vec_loads, int group_m, int splits,
                              hipStream_t stream) {
    SplitK sk;
    sk.splits = mfma_effective_splits(g.K, splits, &sk.k_per);
    sk.ws = nullptr;
    if (sk.splits <= 1) {
        sk.splits = 1;
        sk.k_per = g.K;
        return launch_kernel(g, config, vec_loads, group_m, sk, stream);
    }
    hipError_t e = scratch_acquire(g.scratch, (size_t)sk.splits * g.M * g.N * sizeof(float), stream,
                                   reinterpret_cast<void **>(&sk.ws));
    if (e != hipSuccess) return e;
    e = launch_kernel(g, config, vec_loads, group_m, sk, stream);
    if (e == hipSuccess) {
        const int64_t total = (int64_t)g.M * g.N;
        const bool vec4 = g.N % 4 == 0 && g.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(g.C) % 16 == 0;
        int64_t blocks = ((vec4 ? total / 4 : total) + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        if (blocks < 1) blocks = 1;
        if (vec4)
            hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, g, sk.ws,
                               sk.splits);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, g, sk.ws,
                               sk.splits);
        e = hipGetLastError();
    }
    const hipError_t r = scratch_release(g.scratch, sk.ws, stream);
    return e == hipSuccess ? r : e;
}

hipError_t launch_mfma_large(const GemmArgs &g, bool vec_loads, hipStream_t stream) {
    return launch_mfma_config(g, 0, vec_loads, 8, 1, stream);
}

hipError_t launch_mfma_small(const GemmArgs &g, bool vec_loads, hipStream_t stream) {
    return launch_mfma_config(g, 1, vec_loads, 8, 1, stream);
}

}  // namespace sgemm
