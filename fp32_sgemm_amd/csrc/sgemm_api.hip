// C interface: argument checks, special cases and kernel selection.
//
// The request is the BLAS-style single-precision GEMM C = alpha*A*B + beta*C on
// row-major matrices ("Learn: Optimizing GEMM", section 3; "How a Matmul Kernel
// Gets Fast", section 1).  A vendor library picks among many shape-specialised
// kernels ("Learn: Optimizing GEMM", section 8; "Writing a Fast Matmul in CUDA,
// Step by Step", section "In the real world"); this library picks among its own
// few kernels by shape and operand alignment, on the host, before one launch.
#include <cmath>
#include <cstdint>

#include "gemm_internal.hpp"
#include "sgemm_f32.h"

namespace {

using sgemm::GemmArgs;

int at_least_one(int v) { return v > 1 ? v : 1; }

// Row widths of the stored A and B: A is M x K (K x M when transposed), B is
// K x N (N x K when transposed).
int validate(int ta, int tb, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
             int ldb, const float *C, int ldc) {
    if (ta != 0 && ta != 1) return SGEMM_F32_ERR_TRANS;
    if (tb != 0 && tb != 1) return SGEMM_F32_ERR_TRANS;
    if (M < 0) return 1;
    if (N < 0) return 2;
    if (K < 0) return 3;
    const bool need_ab = M > 0 && N > 0 && K > 0 && alpha != 0.f;
    const bool need_c = M > 0 && N > 0;
    if (need_ab && A == nullptr) return 5;
    if (lda < at_least_one(ta ? M : K)) return 6;
    if (need_ab && B == nullptr) return 7;
    if (ldb < at_least_one(tb ? K : N)) return 8;
    if (need_c && C == nullptr) return 10;
    if (ldc < (N > 1 ? N : 1)) return 11;
    return 0;
}

// The 16-byte-load kernels need 16-byte aligned operands with row strides that
// are multiples of 4 floats, and address one slice of a tile with 32-bit byte
// offsets: the stored rows that one slice touches must span less than 2 GiB
// (128 rows for an operand read along k: A as given, B transposed; 32 rows for
// one read along M or N: B as given, A transposed).
bool slice_fits(bool k_major, int ld) {
    const int64_t limit = (int64_t)1 << 31;
    const int64_t span = k_major ? 127 * (int64_t)ld + 32 : 31 * (int64_t)ld + 128;
    return span * 4 < limit;
}

// Configuration 6 stages slices of 64 values of k: an operand stored along M
// or N then spans 64 stored rows per slice.
bool config_fits(int config, int ta, int tb, int lda, int ldb) {
    if (config != 6) return true;
    const int64_t limit = (int64_t)1 << 31;
    auto fits = [&](int64_t ld) { return (63 * ld + 128) * 4 < limit; };
    return fits(lda) && fits(ldb);
}

bool vec_aligned(int ta, int tb, const float *A, int lda, const float *B, int ldb) {
    const bool aligned = (reinterpret_cast<uintptr_t>(A) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(B) % 16 == 0) && (lda % 4 == 0) && (ldb % 4 == 0);
    return aligned && slice_fits(!ta, lda) && slice_fits(tb, ldb);
}

// Large 128x128 tiles unless they leave most compute units idle and the
// 64x64 tiles give at least one tile per compute unit of the 256.
bool prefer_small_tiles(int M, int N) {
    const int64_t large = sgemm::mfma_large_grid(M, N);
    return large < 256;
}

bool aligned16(const float *A, int lda, const float *B, int ldb) {
    return (reinterpret_cast<uintptr_t>(A) % 16 == 0) && (reinterpret_cast<uintptr_t>(B) % 16 == 0) &&
           (lda % 4 == 0) && (ldb % 4 == 0);
}

// ---------------------------------------------------------------------------
// Tuning table.  The autotuning sweep of "How a Matmul Kernel Gets Fast"
// (section "Kernel 9: autotuning") and the shape-keyed kernel choice of a
// vendor library ("Writing a Fast Matmul in CUDA, Step by Step", section "In
// the real world") become a table from shape classes to an MFMA tile
// configuration, a tile-row grouping and a K split, measured on the GPU by the
// package's tuning script and compiled in.  Class c of an extent x is the first
// c with x <= kClassBound[c]; larger extents use the last class.
// ---------------------------------------------------------------------------
struct TunedEntry {
    signed char config, group_m, splits;
};
constexpr int kNumClasses = 8;
constexpr int kClassBound[kNumClasses] = {64, 128, 256, 512, 1024, 2048, 4096, 8192};

#include "sgemm_tuning_table.inc"   // kHaveTunedTable, kTunedTable[m][n][k]

int shape_class(int x) {
    for (int c = 0; c < kNumClasses; ++c)
        if (x <= kClassBound[c]) return c;
    return kNumClasses - 1;
}

// Bytes of split partials a plan may keep in the stream's workspace.
constexpr int64_t kMaxSplitBytes = (int64_t)1 << 30;

struct Plan {
    int variant;   // sgemm_f32_variant_id that runs
    int config;    // MFMA tile configuration (MFMA variants)
    int group_m;
    int splits;
    int pack = 0;  // operands first copied to aligned scratch rows: 1 = A, 2 = B
};

// Operands that 16-byte loads cannot read take the 4-byte-load tiles; on a
// grid of fewer than 256 of them K is split until about kScalarSplitSlots
// work-groups run, every split at least 256 deep (4096 x 17 x 4096 with ldb =
// 17: 64 tiles of 64 x 64, 157 us in one pass).
constexpr int kScalarSplitSlots = 512;

int scalar_splits(int M, int N, int K, int config) {
    const int64_t tiles = config == 1 ? sgemm::mfma_small_grid(M, N) : sgemm::mfma_large_grid(M, N);
    if (tiles >= 256) return 1;
    int64_t splits = (kScalarSplitSlots + tiles - 1) / tiles;
    if (splits > K / 256) splits = K / 256;
    if (splits > 32) splits = 32;
    while (splits > 1 && splits * M * N * 4 > kMaxSplitBytes) --splits;
    return splits < 1 ? 1 : (int)splits;
}

Plan default_plan(int ta, int tb, int M, int N, int K, const float *A, int lda, const float *B, int ldb) {
    if (sgemm::skinny_form(ta, tb, M, N, K, lda, ldb) >= 0) return Plan{SGEMM_F32_SKINNY, 0, 0, 0};
    const int config = prefer_small_tiles(M, N) ? 1 : 0;
    if (!vec_aligned(ta, tb, A, lda, B, ldb))
        return Plan{SGEMM_F32_MFMA_SCALAR, config, 8, scalar_splits(M, N, K, config)};
    // With 16-byte loads the small tile keeps two slices in flight
    // (configuration 4): one work-group per compute unit or fewer leaves the
    // memory latency to the pipeline alone.
    if (config) return Plan{SGEMM_F32_MFMA_TUNED, 4, 8, 1};
    return Plan{SGEMM_F32_MFMA_LARGE, 0, 8, 1};
}

// Wave quantization of the 128x128 grid.  About kResidentLargeTiles of its
// work-groups are resident at once (two per compute unit on the 256 compute
// units of MI355X), so a grid of T tiles runs ceil(T / 512) rounds, the last
// possibly far from full.  When the tiles fill less than kFillBelow of their
// rounds, the plan moves to 64x64 tiles with two slices in flight (four
// times the tiles, four resident per compute unit, a last round that costs
// far less).  Per-launch timings on MI355X (TFLOP/s, 128x128 -> 64x64 two
// slices ahead, group 8; fill of the 128x128 rounds in brackets): 3000^3
// (0.56) 100.4 -> 128.8, 3072^3 (0.56) 106.9 -> 135.7, 3500^3 (0.77) 103.1
// -> 131.0, 5000 x 5000 x 1000 (0.78) 113.9 -> 122.6, 5120 x 5120 x 2048
// (0.78) 128.1 -> 136.8, 4608 x 4608 x 2048 (0.84) 120.4 -> 133.7, 7168 x 7168
// x 1024 (0.88) 131.1 -> 135.3; and the other way: 4096 x 11008 x 512 (0.90)
// 125.3 / 126.9, 6144 x 6144 x 2048 (0.90) 142.7 / 138.3, 10240 x 10240 x 1024
// (0.96) 139.1 / 136.1, 4096^3 (1.0) 143.1 / 139.4.  A single partial round
// (256 to 511 tiles: some compute units run two work-groups, the others one)
// costs as much as a full one: 2048 x 2560 x 2048 (0.63) 87 -> 123-129, 2304 x
// 2304 x 4096 (0.63) 90 -> 119, 2048 x 3072 x 1024 (0.75) 100 -> 123-128,
// 2560^3 (0.78) 109 -> 123, 2048^3 (0.5) 122-125 -> 127-130; 2816^3 (0.95)
// 131.5 / 130.  The persistent stream-K configuration was slower than the
// 64x64 tiles on the multi-round shapes (e.g. 3000^3 124.1, 5000 x 5000 x 1000
// 115.8), so this rule does not choose it.  The table's octave classes cannot
// express this: the fill depends on the exact tile count.
constexpr int kResidentLargeTiles = 512;
constexpr double kFillBelow = 0.88;

bool rounds_poorly_filled(int M, int N) {
    const int64_t tiles = sgemm::mfma_config_tiles(0, M, N);
    // Fewer than 256 tiles take the small tiles by default (prefer_small_tiles).
    if (tiles < kResidentLargeTiles / 2) return false;
    const int64_t rounds = (tiles + kResidentLargeTiles - 1) / kResidentLargeTiles;
    return (double)tiles < kFillBelow * (double)(rounds * kResidentLargeTiles);
}

Plan quantization_plan(const Plan &p, int M, int N, int K) {
    (void)K;
    if ((p.variant != SGEMM_F32_MFMA_LARGE && p.variant != SGEMM_F32_MFMA_TUNED) || p.config != 0 || p.splits > 1)
        return p;
    if (!rounds_poorly_filled(M, N)) return p;
    return Plan{SGEMM_F32_MFMA_TUNED, 4, 8, 1};
}

// 256x256 tiles (configuration 7) for grids that fill their rounds: one
// work-group per compute unit, so kResidentBigTiles per round.  The fill is
// the share of the rounds' tile area that lies inside C (edge tiles count for
// their inner part), and the 256x256 grid must fill at least kBigFill and
// within kBigMargin of the 128x128 grid's fill (its loop runs about 2-3 %
// faster).  Same-box per-launch medians (TFLOP/s, 128x128 -> 256x256):
// 4096^3 with alpha 1.5, beta -0.5 143.2 -> 147.1, NT 144.6 -> 147.1; 8192^3
// 147.2 -> 149.1; 4096 x 4096 x 1024 136.6 -> 140.4; 4092^3 137.7-139.9 ->
// 141.6, TN 135.4 -> 142.6; 4000^3 (fill 0.95) 131-135 -> 138.5, 4032^3
// (0.97) 136.5 -> 140.8, 3968 x 3968 x 2048 (0.94) 134.0 -> 134.9; and the
// other way 4096 x 11008 x 512 (fill 0.90) 131 -> 120, 6144 x 6144 x 2048
// (0.75) 144 -> 111.
constexpr int kResidentBigTiles = 256;
constexpr double kBigFill = 0.93;
constexpr double kBigMargin = 0.02;

double round_fill(int M, int N, int tile, int per_round) {
    const int64_t tiles = (int64_t)((M + tile - 1) / tile) * ((N + tile - 1) / tile);
    const int64_t rounds = (tiles + per_round - 1) / per_round;
    return (double)M * N / ((double)rounds * per_round * tile * tile);
}

Plan big_tile_plan(const Plan &p, int ta, int tb, int M, int N, int K, const float *A, int lda, const float *B,
                   int ldb) {
    if ((p.variant != SGEMM_F32_MFMA_LARGE && p.variant != SGEMM_F32_MFMA_TUNED) || p.config != 0 || p.splits > 1)
        return p;
    sgemm::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.B = B;
    g.lda = lda; g.ldb = ldb;
    g.trans_a = ta; g.trans_b = tb;
    if (!sgemm::big_tile_fits(g) || sgemm::big_tiles(M, N) < kResidentBigTiles) return p;
    const double fill = round_fill(M, N, 256, kResidentBigTiles);
    if (fill < kBigFill || fill < round_fill(M, N, 128, kResidentLargeTiles) - kBigMargin) return p;
    return Plan{SGEMM_F32_MFMA_TUNED, 7, 4, 1};
}

// The 128x128 grid that remains goes to the kernel of the 256x256 tiles on
// 128x128 tiles (configuration 8: operands copied straight into LDS, two
// work-groups per compute unit) when the operands fit it.  Same-box
// per-launch medians (TFLOP/s, configuration 0 -> 8, NN unless noted): 4096 x 11008 x 512 131.2 -> 133.4, NT 131.6 ->
// 134.2, TN 130.6 -> 131.7; 11008 x 4096 x 512 TT 128.3 -> 131.6; 6144 x 6144
// x 2048 142.5 -> 143.5; 2816^3 132.3 -> 136.8; 8192 x 4096 x 1024 135.5 ->
// 139.5; 16384 x 16384 x 512 132.5 -> 133.8; 3968 x 3968 x 2048 133.7 ->
// 135.8; 5888 x 5888 x 1024 128.9 -> 130.5.  With N not a multiple of 128
// (rows of C not 128-byte aligned, a column of edge tiles) it lost 1-4 % while
// its epilogue stored non-temporally; with plain stores: 6000 x 6000 x 2048
// 135.5 -> 139.3, NT 139.2 -> 139.7, TN 132.6 -> 138.7; 7000 x 7000 x 1024
// 135.0 -> 138.1, NT 137.7 -> 137.5, TN 132.0 -> 137.1; 6100 x 6100 x 1024
// 133.1 -> 138.7, TN 130.1 -> 137.3; 10000 x 10000 x 1024 134.5 -> 136.0;
// 7000 x 7000 x 2048 with alpha 1.5, beta -0.5 136.6 -> 138.7, NT 139.5 ->
// 138.4.  With a K tail (once only the iterations that load the partial
// slice check k): 7000 x 7000 x 1000 130.0 -> 138.4, TN 129.5 -> 137.0;
// 4096 x 4096 x 1000 133.9 -> 138.9; 8192 x 8192 x 1020 139.9 -> 143.1;
// 10000 x 10000 x 1012 132.5 -> 136.3; 3000^3 (forced) 100.4 -> 104.4.
// In the same way the 64x64 grid with two slices in flight (configuration 4)
// without a split goes to that kernel on 64x64 tiles (configuration 9, four
// work-groups per compute unit) for whole 64x64 grids of at most
// kResidentSmallTiles tiles (one round): 1024^3 87.8
// -> 92.5, TN 93.6 -> 101.9; 1536^3 97.6 -> 101.5; 2048^3 TN 135.4 -> 139.1;
// 2048 x 2048 x 1024 127.0 -> 128.0; 512 x 512 x 8192 (no split) 31.8 -> 33.3,
// TN 30.1 -> 33.6; 2048 x 2000 x 2048 122.6 -> 125.7, TN 121.5 -> 127.8; with
// edge tiles (M, N multiples of 4), same box, forced plans: 500 x 2000 x 4096
// 109.0 -> 124.3, 1000^3 94.8 -> 104.1, 700 x 900 x 3000 69.9 -> 79.5, 100 x
// 5000 x 2048 54.4 -> 61.8, 1020^3 98.9 -> 107.1, 2044^3 131.7 -> 135.1, 1500 x
// 1500 x 2000 96.9 -> 100.8, 2000 x 2000 x 8192 134.7 -> 135.5, 1000 x 1000 x
// 256 66.3 -> 66.5 (twelve shapes, none lost).
// Grids of several rounds did not gain: 2560^3 127.5 -> 126.7, TN 126.8 ->
// 128.9; 4608 x 4608 x 2048 135.8 -> 134.9, TN 135.5 -> 138.2; 3008^3 121.4
// -> 109.5, TN 127.8 -> 121.1; and with edge tiles and a K tail 3000^3 130.6
// -> 113.4.  With a K tail: 1024 x 1024 x 1020 84.0 -> 88.0, TN 88.9 -> 96.4;
// 1024 x 1024 x 4092 118.1 -> 124.4, TN 113.7 -> 126.1; 2048 x 1024 x 1000
// 112.6 -> 116.4; 2048 x 2048 x 2044 TN 133.0 -> 137.2, NT 130.7 -> 129.0.
constexpr int64_t kResidentSmallTiles = 1024;
Plan direct_lds_plan(const Plan &p, int ta, int tb, int M, int N, int K, const float *A, int lda,
                     const float *B, int ldb) {
    if ((p.variant != SGEMM_F32_MFMA_LARGE && p.variant != SGEMM_F32_MFMA_TUNED) || p.splits > 1) return p;
    if (p.config != 0 && p.config != 4) return p;
    sgemm::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.B = B;
    g.lda = lda; g.ldb = ldb;
    g.trans_a = ta; g.trans_b = tb;
    if (!sgemm::big_tile_fits(g)) return p;
    if (p.config == 4 && (int64_t)((M + 63) / 64) * ((N + 63) / 64) > kResidentSmallTiles) return p;
    return Plan{SGEMM_F32_MFMA_TUNED, p.config == 0 ? 8 : 9, p.group_m, 1};
}

// 192x192 tiles (configuration 10: the same kernel, one work-group per compute
// unit) for grids of whole rounds of such tiles (at most 6 short of a multiple
// of 256) and K of at least 1024: one round in place of 64x64 or 128x128
// tiles, several in place of 64x64 tiles (the plan for 128x128 grids that
// fill their rounds poorly).  Several rounds, same box, configuration 4 -> 10
// (TFLOP/s): 6144 x 3072 x 2048 140.2 -> 143.6, 6144 x 3072 x 1024 136.4 ->
// 139.5, 4608 x 6144 x 2048 141.1 -> 144.0, 9216 x 3072 x 2048 140.6 ->
// 144.0, 6144 x 4608 x 4096 143.1 -> 145.8, 3072 x 9216 x 1024 137.5 ->
// 140.4; but 4608 x 4608 x 4096 (2.25 rounds) 139.4 -> 109.4, and 6144^3
// (four rounds, configuration 8) 149.3 -> 147.0.  One round, same box
// medians (microseconds, configuration 4 / the automatic plan -> 10, NN, alpha
// 1, beta 0): 3000^3 405.7 -> 394.0; 3072^3 409.8 -> 402.8; 3072 x 3072 x 8192
// 1085.9 -> 1056.8; 1536 x 6144 x 4096 542.8 -> 531.5; 3072 x 3072 x 1024
// 141.1 -> 140.4; 2976^3 388.8 -> 388.4; and the other way 3072 x 2880 x 2048
// (240 tiles) 269.1 -> 270.4, 2880^3 (225) 346.9 -> 376.0, 3584^3 (361, two
// rounds) 678.5 -> 921.6, 4096 x 11008 x 512 339.5 -> 358.5.
constexpr int64_t kRound192Min = 250;
Plan round192_plan(const Plan &p, int ta, int tb, int M, int N, int K, const float *A, int lda, const float *B,
                   int ldb) {
    if ((p.variant != SGEMM_F32_MFMA_LARGE && p.variant != SGEMM_F32_MFMA_TUNED) || p.splits > 1) return p;
    if (p.config != 0 && p.config != 4) return p;
    const int64_t tiles = sgemm::mfma_config_tiles(10, M, N);
    const int64_t rounds = (tiles + kResidentBigTiles - 1) / kResidentBigTiles;
    if (K < 1024 || tiles < rounds * kResidentBigTiles - (kResidentBigTiles - kRound192Min)) return p;
    if (rounds > 1 && p.config != 4) return p;
    sgemm::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.B = B;
    g.lda = lda; g.ldb = ldb;
    g.trans_a = ta; g.trans_b = tb;
    if (!sgemm::big_tile_fits(g)) return p;
    return Plan{SGEMM_F32_MFMA_TUNED, 10, 8, 1};
}

// A 64x64 grid that runs unevenly on the compute units (configuration 9, or
// 4 without a split: the busiest CU holds at least kSplitImbalance times the
// mean number of tiles)
// with K of at least kSplitMinK goes back to configuration 4 with K split in 2
// or 3, whichever spreads the tile-splits more evenly (2 on a tie).  Same-box
// TFLOP/s, configuration 9 -> split: 1152 x 1152 x 4096 88.9 -> 117.5 (3);
// 1152 x 1152 x 2048 86.6 -> 105.4 (3); 1280 x 1280 x 4096 109.2 -> 117.7 (3);
// 1536 x 1536 x 2048 105.1 -> 111.5 (3); 1536 x 1536 x 4096 108.6 -> 128.2
// (3); 1536 x 1536 x 8192 108.9 -> 125.3 (3); 1792 x 1792 x 4096 109.9 ->
// 119.7 (3); 1600 x 1600 x 4096 116.1 -> 121.1 (2); 1536 x 1024 x 4096 105.0
// -> 123.3 (2); 1024 x 1536 x 3072 104.2 -> 119.9 (2); 1280 x 1280 x 2048
// 106.2 -> 106.1 (3); 1536^3 103.9 -> 109.0 (3); 1792^3 108.1 -> 111.7 (3);
// 1600^3 111.2 -> 111.3 (2).  Evenly spread grids lost (1408 x 1408 x 4096,
// 1.06 tiles per CU over the mean, 128.3 -> 121.8; 1664 x 1664 x 4096, 1.14,
// 124.2 -> 120.4), and so did K below 1536 (1280^3 103.2 -> 96.3).  Through
// the automatic plan on another box, against torch's FP32 mm (TFLOP/s):
// 1152 x 1152 x 4096 119.8 / 112.4, 1536 x 1536 x 4096 124.8 / 132.7, 1792 x
// 1792 x 4096 122.0 / 121.7, 1600 x 1600 x 4096 126.9 / 126.0.  The same
// rule on an unsplit configuration-4 grid (extents that keep the
// direct-to-LDS tiles out), same box: 131 x 6000 x 2048 49.6 -> 65.3 (3),
// 1001 x 1500 x 2048 93.9 -> 110.0 (2), 3001 x 700 x 2000 90.0 -> 101.3 (3),
// 601 x 2500 x 4096 98.0 -> 102.6 (3), 255 x 3000 x 4096 84.4 -> 86.1 (2).
constexpr double kSplitImbalance = 1.2;
constexpr int kSplitMinK = 1536;
double cu_imbalance(int64_t units) {
    const double per = (double)units / kResidentBigTiles;
    return std::ceil(per) / per;
}
Plan balance_split_plan(const Plan &p, int M, int N, int K) {
    if (p.variant != SGEMM_F32_MFMA_TUNED || (p.config != 9 && p.config != 4) || p.splits > 1 || K < kSplitMinK)
        return p;
    const int64_t tiles = sgemm::mfma_config_tiles(p.config, M, N);
    if (cu_imbalance(tiles) < kSplitImbalance) return p;
    const int splits = cu_imbalance(3 * tiles) < cu_imbalance(2 * tiles) ? 3 : 2;
    return Plan{SGEMM_F32_MFMA_TUNED, 4, p.group_m, splits};
}

// A 64x64 grid of configuration 9 that is also one round of 250 to 256
// 128x128 tiles (one per compute unit) with K of at least 1024 goes to those
// tiles (configuration 8).  Same-box TFLOP/s, configuration 9 -> 8: 2048^3
// 136.8 -> 139.6; 2048 x 2048 x 4096 138.6 -> 143.2; 1024 x 4096 x 4096
// 139.3 -> 143.2; 4096 x 1024 x 4096 138.7 -> 143.5; 2048 x 2048 x 1024
// 131.7 -> 132.6; with fewer 128x128 tiles configuration 8 leaves CUs idle
// (256 x 4096 x 4096, 64 tiles: 134.1 -> 36.2).
constexpr int64_t kRound128Min = 250;
Plan round128_plan(const Plan &p, int M, int N, int K) {
    if (p.variant != SGEMM_F32_MFMA_TUNED || p.config != 9 || p.splits > 1 || K < 1024) return p;
    const int64_t tiles = sgemm::mfma_config_tiles(8, M, N);
    if (tiles < kRound128Min || tiles > kResidentBigTiles) return p;
    return Plan{SGEMM_F32_MFMA_TUNED, 8, p.group_m, 1};
}

// The automatic choice: the M <= 32 kernel and the 4-byte-load kernels as in
// default_plan; for 16-byte-aligned operands the tuning table's entry for the
// shape class when there is one, then the switch to 64x64 tiles for 128x128
// grids that fill their rounds poorly, to 256x256 tiles for grids that fill
// theirs, to 192x192 tiles for grids of whole rounds of them, from the 128x128
// and 64x64 kernels to configurations 8 and 9, from an unevenly spread
// configuration 9 back to a K split, and from a configuration 9 grid that is
// one round of 128x128 tiles to those (reported as SGEMM_F32_MFMA_TUNED when
// the plan differs from the default).
// Transposed operands use the same entries.
Plan auto_plan(int ta, int tb, int M, int N, int K, const float *A, int lda, const float *B, int ldb);

// An operand read along M or N whose extent is not a multiple of 4 (B as
// given with N % 4 != 0, A transposed with M % 4 != 0) has 16-byte groups
// straddling the edge of the last tiles, which load them element by element
// on every slice; on a grid of one round those tiles set the time.  The
// unsplit 64x64 grid with two slices in flight then splits K: in 3 up to 256
// tiles, in 2 up to 512, with K of at least 2048 (same box, TFLOP/s, 1 -> 3
// splits: 512 x 2047 x 4096 66.1 -> 113.2, 1000 x 1001 x 2048 60.7 -> 95.4,
// 300 x 3001 x 4096 56.2 -> 87.9; 2048 x 1023 x 2048, 512 tiles, 96.7 -> 105.3
// with 2; with K = 1024 or about 1000 tiles splits lost: 1024 x 1023 x 1024
// 86.9 -> 73.3, 4000 x 999 x 2048 112.8 -> 105.1).
Plan straddle_split_plan(const Plan &p, int ta, int tb, int M, int N, int K) {
    if (p.variant != SGEMM_F32_MFMA_TUNED || p.config != 4 || p.splits > 1 || K < 2048) return p;
    const bool straddle = (!tb && N % 4 != 0) || (ta && M % 4 != 0);
    const int64_t tiles = sgemm::mfma_small_grid(M, N);
    if (!straddle || tiles > 512) return p;
    Plan q = p;
    q.splits = tiles <= 256 ? 3 : 2;
    if ((int64_t)q.splits * M * N * 4 > kMaxSplitBytes) return p;
    return q;
}

// Operands that 16-byte loads cannot take, on a product of at least 2^32
// FLOP: the operand (or both) is first copied into scratch rows padded to a
// multiple of 4 floats, and the product runs the plan aligned operands get
// (not stream-K), when the copies and that plan's split partials fit in
// SGEMM_F32_NOALLOC_SCRATCH_BYTES together (so the allocation-free entry
// point takes the same plan); one acquisition holds both, the partials after
// the copies.  Per call, 4-byte
// loads -> copies and 64x64 tiles with two slices in flight (odd extents keep
// the direct-to-LDS tiles out): 2047^3 195.7 -> 167.4 us, 3001 x 2001 x 1001
// 154.9 -> 121.2, 2048 x 2048 x 2047 154.6 -> 136.4; 1023^3 lost (42.6 ->
// 47.3), hence the lower bound.
constexpr int64_t kPackMinFlop = (int64_t)1 << 32;
constexpr int64_t kPackMaxBytes = SGEMM_F32_NOALLOC_SCRATCH_BYTES;

struct PackShape {
    int a_rows, a_cols, b_rows, b_cols;
    int64_t lda2, ldb2, a_bytes, b_bytes;   // a_bytes, b_bytes rounded up to 256
};

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

PackShape pack_shape(int pack, int ta, int tb, int M, int N, int K, int64_t lda, int64_t ldb) {
    PackShape s;
    s.a_rows = ta ? K : M;
    s.a_cols = ta ? M : K;
    s.b_rows = tb ? N : K;
    s.b_cols = tb ? K : N;
    s.lda2 = (pack & 1) ? round_up(s.a_cols, 4) : lda;
    s.ldb2 = (pack & 2) ? round_up(s.b_cols, 4) : ldb;
    s.a_bytes = (pack & 1) ? round_up((int64_t)s.a_rows * s.lda2 * 4, 256) : 0;
    s.b_bytes = (pack & 2) ? round_up((int64_t)s.b_rows * s.ldb2 * 4, 256) : 0;
    return s;
}

// Split partials of an MFMA plan on packed operands (bytes; 0 without a split).
int64_t packed_partial_bytes(const Plan &p, int M, int N, int K) {
    if (p.splits <= 1) return 0;
    int k_per = 0;
    const int splits = sgemm::mfma_effective_splits(K, p.splits, &k_per);
    return splits > 1 ? round_up((int64_t)splits * M * N * 4, 256) : 0;
}

Plan pack_plan(const Plan &d, int ta, int tb, int M, int N, int K, const float *A, int lda, const float *B, int ldb) {
    if (2 * (int64_t)M * N * K < kPackMinFlop) return d;
    const bool pa = !(aligned16(A, lda, A, 0) && slice_fits(!ta, lda));
    const bool pb = !(aligned16(B, ldb, B, 0) && slice_fits(tb, ldb));
    if (!pa && !pb) return d;
    const int pack = (pa ? 1 : 0) | (pb ? 2 : 0);
    const PackShape s = pack_shape(pack, ta, tb, M, N, K, lda, ldb);
    if (s.lda2 > INT32_MAX || s.ldb2 > INT32_MAX || s.a_bytes + s.b_bytes > kPackMaxBytes) return d;
    const float *aligned_stand_in = reinterpret_cast<const float *>((uintptr_t)256);
    Plan p = auto_plan(ta, tb, M, N, K, pa ? aligned_stand_in : A, (int)s.lda2, pb ? aligned_stand_in : B,
                       (int)s.ldb2);
    if (p.variant == SGEMM_F32_MFMA_SCALAR || p.variant == SGEMM_F32_SKINNY || p.variant == SGEMM_F32_VALU ||
        p.config == 5 || s.a_bytes + s.b_bytes + packed_partial_bytes(p, M, N, K) > kPackMaxBytes)
        return d;
    p.pack = pack;
    return p;
}

Plan auto_plan(int ta, int tb, int M, int N, int K, const float *A, int lda, const float *B, int ldb) {
    const Plan d = default_plan(ta, tb, M, N, K, A, lda, B, ldb);
    if (d.variant == SGEMM_F32_SKINNY) return d;
    if (d.variant == SGEMM_F32_MFMA_SCALAR) return pack_plan(d, ta, tb, M, N, K, A, lda, B, ldb);
    Plan p = d;
    if (kHaveTunedTable) {
        const TunedEntry e = kTunedTable[shape_class(M)][shape_class(N)][shape_class(K)];
        if (e.config >= 0 && e.config < sgemm::kNumMfmaConfigs && e.group_m >= 1 && e.splits >= 1 &&
            config_fits(e.config, ta, tb, lda, ldb)) {
            int k_per = 0;
            int splits = sgemm::mfma_effective_splits(K, e.splits, &k_per);
            if ((int64_t)splits * M * N * 4 > kMaxSplitBytes) splits = 1;
            p = Plan{SGEMM_F32_MFMA_TUNED, e.config, e.group_m, splits};
            if (p.config == d.config && p.group_m == d.group_m && p.splits <= 1) p = d;
        }
    }
    p = big_tile_plan(quantization_plan(p, M, N, K), ta, tb, M, N, K, A, lda, B, ldb);
    p = round192_plan(p, ta, tb, M, N, K, A, lda, B, ldb);
    p = balance_split_plan(direct_lds_plan(p, ta, tb, M, N, K, A, lda, B, ldb), M, N, K);
    return straddle_split_plan(round128_plan(p, M, N, K), ta, tb, M, N, K);
}

int to_status(hipError_t e) { return e == hipSuccess ? 0 : -static_cast<int>(e); }

constexpr int64_t kMaxGrid = 0x7fffffff;

// One MFMA launch (plus the split reduction) after its plan is known.
int run_mfma(const GemmArgs &g, int config, bool vec, int group_m, int splits, hipStream_t stream) {
    if (!vec && !sgemm::mfma_config_scalar_ok(config)) return SGEMM_F32_ERR_NOT_APPLICABLE;
    if (!config_fits(config, g.trans_a, g.trans_b, g.lda, g.ldb)) return SGEMM_F32_ERR_NOT_APPLICABLE;
    if (config >= 7 && !(sgemm::big_tile_fits(g) && sgemm::big_tile_c_fits(g.ldc)))
        return SGEMM_F32_ERR_NOT_APPLICABLE;
    int k_per = 0;
    const int eff = sgemm::mfma_config_splits_ok(config) ? sgemm::mfma_effective_splits(g.K, splits, &k_per) : 1;
    if (sgemm::mfma_config_tiles(config, g.M, g.N) * eff > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
    if (eff > 1 && (int64_t)eff * g.M * g.N * 4 > kMaxSplitBytes) return SGEMM_F32_ERR_TOO_LARGE;
    return to_status(sgemm::launch_mfma_config(g, config, vec, group_m, eff, stream));
}

GemmArgs make_args(int ta, int tb, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                   int ldb, float beta, float *C, int ldc) {
    GemmArgs g;
    g.M = M; g.N = N; g.K = K;
    g.alpha = alpha; g.beta = beta;
    g.A = A; g.B = B; g.C = C;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc;
    g.trans_a = ta; g.trans_b = tb;
    return g;
}

// Scratch bytes of a plan (0 for plans without a split), or -1 when the
// occupancy query of the stream-K plan fails.
int64_t plan_scratch_bytes(const Plan &p, const GemmArgs &g) {
    if (p.pack) {   // the copies, then the plan's split partials
        const PackShape s = pack_shape(p.pack, g.trans_a, g.trans_b, g.M, g.N, g.K, g.lda, g.ldb);
        return s.a_bytes + s.b_bytes + packed_partial_bytes(p, g.M, g.N, g.K);
    }
    if (p.variant == SGEMM_F32_SKINNY) return sgemm::skinny_scratch_bytes(g);
    if (p.variant == SGEMM_F32_VALU) return 0;
    int config = p.variant == SGEMM_F32_MFMA_TUNED ? p.config : (p.variant == SGEMM_F32_MFMA_SMALL ? 1 : 0);
    if (p.variant == SGEMM_F32_MFMA_SCALAR) config = prefer_small_tiles(g.M, g.N) ? 1 : 0;
    const int splits = p.variant == SGEMM_F32_MFMA_TUNED || p.variant == SGEMM_F32_MFMA_SCALAR ? p.splits : 1;
    int64_t bytes = 0;
    if (sgemm::mfma_config_scratch_bytes(g, config, splits, &bytes) != hipSuccess) return -1;
    return bytes;
}

int dispatch(const Plan &p, const GemmArgs &g, bool vec, bool plain, hipStream_t stream);

int run(int variant, int ta, int tb, int M, int N, int K, float alpha, const float *A, int lda,
        const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream,
        const sgemm::Scratch &scratch = sgemm::Scratch{}) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    const int bad = validate(ta, tb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (bad) return bad;
    if (M == 0 || N == 0) return 0;

    GemmArgs g = make_args(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    g.scratch = scratch;
    if (alpha == 0.f || K == 0) {
        if ((int64_t)M * N > (int64_t)1 << 62) return SGEMM_F32_ERR_TOO_LARGE;
        return to_status(sgemm::launch_scale_c(g, stream));
    }

    bool vec = vec_aligned(ta, tb, A, lda, B, ldb);
    const bool plain = !ta && !tb;
    Plan p{variant, 0, 8, 1};
    if (variant == SGEMM_F32_AUTO) {
        p = auto_plan(ta, tb, M, N, K, A, lda, B, ldb);
    } else if (variant == SGEMM_F32_MFMA_TUNED) {
        if (!vec) return SGEMM_F32_ERR_NOT_APPLICABLE;
        p = auto_plan(ta, tb, M, N, K, A, lda, B, ldb);
    }
    // The plan does not see C: a row stride of C too wide for the 32-bit
    // offsets of configurations 7-9 keeps the register-staged kernels.
    if ((p.config == 7 || p.config == 8 || p.config == 10) && !sgemm::big_tile_c_fits(ldc))
        p = Plan{SGEMM_F32_MFMA_LARGE, 0, 8, 1, p.pack};
    if (p.config == 9 && !sgemm::big_tile_c_fits(ldc)) p = Plan{SGEMM_F32_MFMA_TUNED, 4, p.group_m, 1, p.pack};
    if (scratch.fixed != nullptr) {
        // A fixed scratch region: refuse, before anything is enqueued, a plan
        // that needs more of it than there is.
        const int64_t need = plan_scratch_bytes(p, g);
        if (need < 0 || need > (int64_t)scratch.fixed_bytes) return SGEMM_F32_ERR_SCRATCH;
    }
    void *pack_ws = nullptr;
    if (p.pack) {
        // Copy the operands that 16-byte loads cannot take into aligned rows
        // of the call's scratch, in stream order before the product.
        const PackShape sh = pack_shape(p.pack, ta, tb, M, N, K, lda, ldb);
        const int64_t copies = sh.a_bytes + sh.b_bytes;
        const int64_t partials = packed_partial_bytes(p, M, N, K);
        hipError_t e = sgemm::scratch_acquire(scratch, (size_t)(copies + partials), stream, &pack_ws);
        if (e != hipSuccess) return to_status(e);
        float *base = static_cast<float *>(pack_ws);
        // The plan's own scratch: the rest of the same block, handed to it as
        // a fixed region (a second acquisition on this stream could return
        // the same cached block).
        if (partials > 0) {
            g.scratch.fixed = static_cast<char *>(pack_ws) + copies;
            g.scratch.fixed_bytes = (size_t)partials;
        }
        if (p.pack & 1) {
            e = sgemm::launch_pack_rows(A, lda, sh.a_rows, sh.a_cols, base, sh.lda2, stream);
            g.A = base;
            g.lda = sh.lda2;
        }
        if (e == hipSuccess && (p.pack & 2)) {
            float *bp = base + sh.a_bytes / 4;
            e = sgemm::launch_pack_rows(B, ldb, sh.b_rows, sh.b_cols, bp, sh.ldb2, stream);
            g.B = bp;
            g.ldb = sh.ldb2;
        }
        if (e != hipSuccess) {
            sgemm::scratch_release(scratch, pack_ws, stream);
            return to_status(e);
        }
        vec = true;
    }
    const int st = dispatch(p, g, vec, plain, stream);
    if (pack_ws != nullptr) {
        const hipError_t r = sgemm::scratch_release(scratch, pack_ws, stream);
        if (st == 0 && r != hipSuccess) return to_status(r);
    }
    return st;
}

// Runs a plan on the call's arguments (operands already packed where the plan says so).
int dispatch(const Plan &p, const GemmArgs &g, bool vec, bool plain, hipStream_t stream) {
    const int M = g.M, N = g.N, K = g.K, ta = g.trans_a, tb = g.trans_b;
    const int64_t lda = g.lda, ldb = g.ldb;
    switch (p.variant) {
        case SGEMM_F32_MFMA_LARGE:
            if (!vec) return SGEMM_F32_ERR_NOT_APPLICABLE;
            return run_mfma(g, 0, true, 8, 1, stream);
        case SGEMM_F32_MFMA_SMALL:
            if (!vec) return SGEMM_F32_ERR_NOT_APPLICABLE;
            return run_mfma(g, 1, true, 8, 1, stream);
        case SGEMM_F32_MFMA_TUNED:
            return run_mfma(g, p.config, vec, p.group_m, p.splits, stream);
        case SGEMM_F32_MFMA_SCALAR:
            return run_mfma(g, prefer_small_tiles(M, N) ? 1 : 0, false, 8, p.splits, stream);
        case SGEMM_F32_VALU:
            if (!plain) return SGEMM_F32_ERR_NOT_APPLICABLE;
            if (sgemm::valu_grid(M, N) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_valu(g, vec, stream));
        case SGEMM_F32_SKINNY:
            if (sgemm::skinny_form(ta, tb, M, N, K, lda, ldb) < 0) return SGEMM_F32_ERR_NOT_APPLICABLE;
            if (sgemm::skinny_grid(g) > kMaxGrid) return SGEMM_F32_ERR_TOO_LARGE;
            return to_status(sgemm::launch_skinny(g, aligned16(g.A, (int)lda, g.B, (int)ldb), stream));
        default:
            return SGEMM_F32_ERR_VARIANT;
    }
}

bool flags_ok(int ta, int tb) { return (ta == 0 || ta == 1) && (tb == 0 || tb == 1); }

}  // namespace

namespace sgemm {

int run_auto_with_scratch(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                          float beta, float *C, int ldc, hipStream_t stream, const Scratch &scratch) {
    return run(SGEMM_F32_AUTO, 0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, scratch);
}

}  // namespace sgemm

extern "C" {

int sgemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
              float beta, float *C, int ldc, hipStream_t stream) {
    return run(SGEMM_F32_AUTO, 0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_variant(int variant, int M, int N, int K, float alpha, const float *A, int lda,
                      const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(variant, 0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_select(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                     int ldb) {
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.f) return 0;
    return auto_plan(0, 0, M, N, K, A, lda, B, ldb).variant;
}

int sgemm_f32_ex(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A, int lda,
                 const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return run(SGEMM_F32_AUTO, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_ex_variant(int variant, int trans_a, int trans_b, int M, int N, int K, float alpha,
                         const float *A, int lda, const float *B, int ldb, float beta, float *C, int ldc,
                         hipStream_t stream) {
    return run(variant, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_f32_ex_select(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A, int lda,
                        const float *B, int ldb) {
    if (!flags_ok(trans_a, trans_b)) return 0;
    if (M <= 0 || N <= 0 || K <= 0 || alpha == 0.f) return 0;
    return auto_plan(trans_a, trans_b, M, N, K, A, lda, B, ldb).variant;
}

int sgemm_f32_ex_plan(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A, int lda,
                      const float *B, int ldb, int *variant, int *config, int *group_m, int *splits) {
    if (variant == nullptr || config == nullptr || group_m == nullptr || splits == nullptr)
        return SGEMM_F32_ERR_CONFIG;
    *variant = *config = *group_m = *splits = 0;
    if (!flags_ok(trans_a, trans_b)) return SGEMM_F32_ERR_TRANS;
    if (M < 0) return 1;
    if (N < 0) return 2;
    if (K < 0) return 3;
    if (M == 0 || N == 0 || K == 0 || alpha == 0.f) return 0;
    const Plan p = auto_plan(trans_a, trans_b, M, N, K, A, lda, B, ldb);
    *variant = p.variant;
    if (p.variant == SGEMM_F32_SKINNY || p.variant == SGEMM_F32_VALU) return 0;
    *config = p.config;
    *group_m = p.group_m;
    int k_per = 0;
    *splits = sgemm::mfma_effective_splits(K, p.splits, &k_per);
    return 0;
}

int sgemm_f32_ex_config(int config, int group_m, int splits, int trans_a, int trans_b, int M, int N, int K,
                        float alpha, const float *A, int lda, const float *B, int ldb, float beta, float *C,
                        int ldc, hipStream_t stream) {
    if (config < 0 || config >= sgemm::kNumMfmaConfigs || group_m < 1 || group_m > 64 || splits < 1 ||
        splits > 64 || (splits > 1 && !sgemm::mfma_config_splits_ok(config)))
        return SGEMM_F32_ERR_CONFIG;
    const int bad = validate(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (bad) return bad;
    if (M == 0 || N == 0) return 0;
    const GemmArgs g = make_args(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    if (alpha == 0.f || K == 0) return to_status(sgemm::launch_scale_c(g, stream));
    return run_mfma(g, config, vec_aligned(trans_a, trans_b, A, lda, B, ldb), group_m, splits, stream);
}

int sgemm_f32_tuning_table_present(void) { return kHaveTunedTable ? 1 : 0; }

const char *sgemm_f32_config_name(int config) {
    switch (config) {
        case 0: return "128x128";
        case 1: return "64x64";
        case 2: return "128x64";
        case 3: return "64x128";
        case 4: return "64x64_pf2";
        case 5: return "128x128_streamk";
        case 6: return "64x64_bk64";
        case 7: return "256x256";
        case 8: return "128x128_dl";
        case 9: return "64x64_dl";
        case 10: return "192x192_dl";
        default: return nullptr;
    }
}

const char *sgemm_f32_variant_name(int variant) {
    switch (variant) {
        case SGEMM_F32_AUTO: return "auto";
        case SGEMM_F32_MFMA_LARGE: return "mfma_large";
        case SGEMM_F32_MFMA_SMALL: return "mfma_small";
        case SGEMM_F32_VALU: return "valu";
        case SGEMM_F32_SKINNY: return "skinny";
        case SGEMM_F32_MFMA_SCALAR: return "mfma_scalar";
        case SGEMM_F32_MFMA_TUNED: return "mfma_tuned";
        default: return nullptr;
    }
}

int sgemm_f32_version(void) { return 300; }

}  // extern "C"
