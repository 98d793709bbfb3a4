/*
 * sgemm_f32.h -- C interface of the single-precision GEMM library for AMD
 * Instinct MI355X (gfx950).
 *
 * Operation ("Learn: Optimizing GEMM", section 3 "Rung 0 -- Naive (recap)",
 * whose listing header states the operation and the three row-major shapes;
 * "How a Matmul Kernel Gets Fast", section 1 "The problem, and what cuBLAS is",
 * on the two scalars):
 *
 *     C = alpha * A * B + beta * C
 *
 * A is M x K, B is K x N, C is M x N, every matrix row-major with an explicit
 * row stride (leading dimension) in elements:
 *
 *     A(i, k) = A[i * lda + k],  B(k, j) = B[k * ldb + j],  C(i, j) = C[i * ldc + j]
 *
 * ("CUDA Matrix Multiplication Optimization: From Naive to Near-cuBLAS",
 * section "Why Naive is Cache-Hostile", addresses element (i, j) as
 * base + i * stride + j; the pages fix the strides to K and N, this interface
 * takes them as arguments.)
 *
 * Arithmetic is IEEE single precision throughout: FP32 products accumulated in
 * FP32 on the matrix cores (or on the vector ALUs in the comparison variant).
 * The summation order over k is not specified; results agree with a float64
 * evaluation to within 2e-5 * (|alpha| * (|A|*|B|)_ij + |beta| * |C_ij|), and are
 * exact whenever every partial sum is exactly representable in FP32 (e.g. small
 * integers).
 *
 * Ownership and execution:
 *   - A, B and C are device pointers owned by the caller.  The library never
 *     frees or retains them.  C must not overlap A or B.
 *   - The work is enqueued on `stream` (0 = the null stream) and the call
 *     returns without waiting for it.  No host or device synchronisation.
 *   - The functions hold no per-call state and may be called from several host
 *     threads at once.
 *   - Device memory (see sgemm_f32_noalloc for the form that allocates
 *     nothing): none unless the reduction over K is split across
 *     work-groups (the streaming kernels, MFMA plans with splits > 1 from the
 *     tuning table or sgemm_f32_ex_config, and the stream-K configuration)
 *     or the automatic choice copies misaligned operands to aligned rows
 *     (at most 64 MiB).  Such a call needs scratch (at most splits * M * N
 *     floats, 1 GiB cap for MFMA plans), taken from a memory pool the library creates on the first
 *     such call on a device (it keeps up to 1 GiB of freed memory and lives
 *     until the process ends):
 *       - outside graph capture, up to 64 MiB, on one of the first 8 streams
 *         (per device) that need scratch: a block the library keeps for that
 *         stream until the process ends, reused by every later call on it
 *         (stream order serialises them) and grown in stream order when a
 *         call needs more.  A block never serves another stream.  A stream
 *         handle must not name a new stream while work on the old one that
 *         used it is pending (destroying a HIP stream waits for its work);
 *       - otherwise (graph capture, larger requests, further streams): in
 *         stream order, hipMallocFromPoolAsync on `stream` before the call's
 *         kernels and hipFreeAsync after them, which graph capture records.
 *     Either way, calls on different streams never share scratch.
 *
 * Special cases:
 *   - M == 0 or N == 0: nothing is done, returns 0.
 *   - alpha == 0 or K == 0: C = beta * C, A and B are not read.
 *   - beta == 0: C is output only and is never read (NaN or garbage in C does
 *     not propagate).
 *
 * Return value:
 *     0                      success (work enqueued)
 *     1, 2, 3                M, N, K negative
 *     5, 7, 10               A, B, C is NULL although it must be accessed
 *     6, 8, 11               lda < max(1, K), ldb < max(1, N), ldc < max(1, N)
 *     SGEMM_F32_ERR_VARIANT  (sgemm_f32_variant only) unknown variant number
 *     SGEMM_F32_ERR_NOT_APPLICABLE  (sgemm_f32_variant only) the forced variant
 *                            cannot run this shape or alignment
 *     SGEMM_F32_ERR_TOO_LARGE  the tile grid exceeds the launch limits
 *     SGEMM_F32_ERR_TRANS    (the _ex functions) a transpose flag other than 0 or 1
 *     SGEMM_F32_ERR_CONFIG   (sgemm_f32_ex_config, sgemm_f32_ex_plan) a configuration,
 *                            grouping or split count out of range, or a NULL output
 *     SGEMM_F32_ERR_SCRATCH  (sgemm_f32_noalloc) the plan needs more scratch than
 *                            the fixed region holds; nothing was enqueued
 *     < 0                    -(hipError_t) reported by the HIP runtime for the
 *                            launch; the contents of C are then unspecified
 * Nothing is printed and no exception crosses the interface.
 */
#ifndef SGEMM_F32_H
#define SGEMM_F32_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_F32_ERR_VARIANT 20
#define SGEMM_F32_ERR_NOT_APPLICABLE 21
#define SGEMM_F32_ERR_TOO_LARGE 22
#define SGEMM_F32_ERR_TRANS 23
#define SGEMM_F32_ERR_CONFIG 24
#define SGEMM_F32_ERR_SCRATCH 25

/* Size of the fixed scratch region that sgemm_f32_noalloc uses on each device. */
#define SGEMM_F32_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Kernel variants that sgemm_f32_variant can force. */
enum sgemm_f32_variant_id {
    SGEMM_F32_AUTO = 0,           /* the same selection sgemm_f32 makes */
    SGEMM_F32_MFMA_LARGE = 1,     /* FP32 MFMA, 128x128 block tile */
    SGEMM_F32_MFMA_SMALL = 2,     /* FP32 MFMA, 64x64 block tile (small shapes) */
    SGEMM_F32_VALU = 3,           /* FP32 FMA on the vector ALUs, 128x128 tile, 8x8 per thread */
    SGEMM_F32_SKINNY = 4,         /* FP32 MFMA streaming kernels: M <= 32 (plain form), or
                                     M <= 16 with B transposed, or N <= 16 with A as given */
    SGEMM_F32_MFMA_SCALAR = 5,    /* FP32 MFMA with 4-byte loads: any alignment and stride (the
                                     automatic choice splits K on grids of fewer than 256 tiles;
                                     on products of at least 2^32 FLOP it copies such operands,
                                     up to 64 MiB, to aligned scratch rows and runs the plan
                                     aligned operands get) */
    SGEMM_F32_MFMA_TUNED = 6,     /* FP32 MFMA with the automatic plan: the tuning table's,
                                     64x64 tiles with two slices in flight, 256x256 tiles, or
                                     128x128 or 64x64 tiles loaded straight into LDS (16-byte
                                     loads) */
    SGEMM_F32_NUM_VARIANTS = 7
};

/* MFMA tile configurations (sgemm_f32_ex_config, sgemm_f32_ex_plan). */
enum sgemm_f32_config_id {
    SGEMM_F32_CFG_128x128 = 0,    /* the SGEMM_F32_MFMA_LARGE tile */
    SGEMM_F32_CFG_64x64 = 1,      /* the SGEMM_F32_MFMA_SMALL tile */
    SGEMM_F32_CFG_128x64 = 2,     /* 16-byte loads only */
    SGEMM_F32_CFG_64x128 = 3,     /* 16-byte loads only */
    SGEMM_F32_CFG_64x64_PF2 = 4,  /* 64x64, two slices in flight; 16-byte loads only */
    SGEMM_F32_CFG_128x128_STREAMK = 5, /* 128x128, persistent with stream-K; 16-byte loads only */
    SGEMM_F32_CFG_64x64_BK64 = 6, /* 64x64, slices of 64, two in flight; 16-byte loads only */
    SGEMM_F32_CFG_256x256 = 7,    /* 256x256, one work-group per CU, operands loaded straight into
                                     LDS; K and the extent of an operand read along M or N
                                     multiples of 4 (edge tiles read zeros past the matrices),
                                     16-byte loads, no K split, group_m ignored
                                     (4 is used) */
    SGEMM_F32_CFG_128x128_DL = 8, /* 128x128 by the kernel of configuration 7, two work-groups per
                                     CU; its conditions, no K split */
    SGEMM_F32_CFG_64x64_DL = 9,   /* 64x64 by the kernel of configuration 7, four work-groups per
                                     CU; its conditions, no K split */
    SGEMM_F32_CFG_192x192_DL = 10, /* 192x192 by the kernel of configuration 7, one work-group per
                                      CU; its conditions, no K split */
    SGEMM_F32_NUM_CONFIGS = 11
};

/*
 * C = alpha * A * B + beta * C on `stream` (see above).
 * M, N, K: matrix sizes (>= 0).  alpha, beta: host scalars, by value.
 * A: device, M x K, row stride lda.  B: device, K x N, row stride ldb.
 * C: device, M x N, row stride ldc, read (if beta != 0) and written.
 */
int sgemm_f32(int M, int N, int K, float alpha,
              const float *A, int lda, const float *B, int ldb,
              float beta, float *C, int ldc, hipStream_t stream);

/*
 * sgemm_f32 for callers that cannot allocate device memory: code under graph
 * capture that must not record allocations, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, validation, special cases, kernel
 * plan and results (bit for bit) as sgemm_f32.  It calls no hipMalloc,
 * hipMallocAsync or hipFree: the plans that need scratch (the streaming kernels' split,
 * tuned split-K plans) use a fixed region of
 * SGEMM_F32_NOALLOC_SCRATCH_BYTES (64 MiB) in the library's device memory,
 * one per device, present from the library's loading on that device until
 * the process ends.  The first call on a device looks up that region's
 * address (hipGetSymbolAddress, no allocation).
 *
 * The region is shared by every sgemm_f32_noalloc call on the device and keeps
 * the last call's contents (nothing in it needs to start at zero): calls that
 * overlap in time on one device (on different streams, or from several host
 * threads without ordering) race on it and give undefined results.  Order
 * them, for example by issuing them on one stream.  A plan that needs more
 * than the region holds returns SGEMM_F32_ERR_SCRATCH without enqueueing
 * anything; C is then unchanged.
 */
int sgemm_f32_noalloc(int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      float beta, float *C, int ldc, hipStream_t stream);

/*
 * The same operation computed by one forced kernel variant, for comparisons
 * between variants and for tests.  Arguments after `variant` are those of
 * sgemm_f32.  Returns SGEMM_F32_ERR_NOT_APPLICABLE when the variant cannot
 * handle the request (SGEMM_F32_SKINNY on a shape none of its forms covers; a vector-load variant with
 * a pointer not 16-byte aligned, lda or ldb not a multiple of 4, or row strides
 * so large that 128 rows of A or 32 rows of B span 2 GiB or more).
 */
int sgemm_f32_variant(int variant, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      float beta, float *C, int ldc, hipStream_t stream);

/*
 * The variant sgemm_f32 would use for these arguments (an
 * sgemm_f32_variant_id), or 0 when it would launch no GEMM kernel (empty
 * output, or alpha == 0 / K == 0 which only scales C).  Host only; no HIP call.
 */
int sgemm_f32_select(int M, int N, int K, float alpha,
                     const float *A, int lda, const float *B, int ldb);

/*
 * Transposed operands ("Writing a Fast Matmul in CUDA, Step by Step", section
 * "In the real world": the library the pages compare against takes every
 * transpose of its operands, and the "nn" in its kernel names marks the form
 * with neither transposed):
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * op(A) is M x K and op(B) is K x N; C is M x N row-major as above.
 *   trans_a == 0: A is stored M x K, op(A)(i, k) = A[i * lda + k], lda >= max(1, K)
 *   trans_a == 1: A is stored K x M, op(A)(i, k) = A[k * lda + i], lda >= max(1, M)
 *   trans_b == 0: B is stored K x N, op(B)(k, j) = B[k * ldb + j], ldb >= max(1, N)
 *   trans_b == 1: B is stored N x K, op(B)(k, j) = B[j * ldb + k], ldb >= max(1, K)
 * Any other flag value returns SGEMM_F32_ERR_TRANS.  Everything else (special
 * cases, ownership, stream, accuracy, return codes) is as for sgemm_f32, and
 * sgemm_f32_ex(0, 0, ...) is sgemm_f32(...).
 *
 * Column-major callers: a column-major C = op(A) * op(B) is, read row-major,
 * C^T = op(B)^T * op(A)^T, so it is
 *     sgemm_f32_ex(tb, ta, N, M, K, alpha, B, ldb, A, lda, beta, C, ldc, stream)
 * with the column-major leading dimensions.
 *
 * Transposed operands run on the MFMA variants (SGEMM_F32_MFMA_LARGE, _SMALL,
 * _SCALAR); SGEMM_F32_VALU takes neither operand transposed and returns
 * SGEMM_F32_ERR_NOT_APPLICABLE otherwise.  SGEMM_F32_SKINNY (and the automatic
 * choice) streams the large operand when its rows run along K: B transposed
 * with M <= 16 (NT, TT), or A as given with N <= 16 (NN, NT; C is then
 * written through its transpose); A transposed with B as given has no
 * streaming form.  Its offsets are 32-bit: 32 rows of the streamed operand,
 * and all of the small one, must span less than 2 GiB.  For the
 * 16-byte-load variants the stored rows one slice touches must span less than
 * 2 GiB: 128 rows of an operand stored along K (A as given, B transposed) and
 * 32 rows of one stored along M or N (B as given, A transposed).
 */
int sgemm_f32_ex(int trans_a, int trans_b, int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb,
                 float beta, float *C, int ldc, hipStream_t stream);

/* sgemm_f32_variant with transposed operands. */
int sgemm_f32_ex_variant(int variant, int trans_a, int trans_b, int M, int N, int K,
                         float alpha, const float *A, int lda, const float *B, int ldb,
                         float beta, float *C, int ldc, hipStream_t stream);

/* sgemm_f32_select with transposed operands (0 for invalid flags as well). */
int sgemm_f32_ex_select(int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const float *A, int lda, const float *B, int ldb);

/*
 * Tuned selection.  Tiling parameters are tuned per problem shape ("How a
 * Matmul Kernel Gets Fast", section "Kernel 9: autotuning"; the vendor library
 * chooses among shape-specialised kernels, "Writing a Fast Matmul in CUDA, Step
 * by Step", section "In the real world").  The library carries a table from
 * shape classes of (M, N, K) (class bounds 64, 128, ..., 8192 per extent) to a
 * plan: a tile configuration, a tile-row grouping of the work-group order and
 * a split of K over work-groups.  The table is measured on the GPU by the
 * package's tuning script (fp32_sgemm_amd/tune.py) and compiled in; for
 * 16-byte-aligned operands sgemm_f32 and sgemm_f32_ex follow it (other cases as
 * before).  A split plan sums its partials in split order, so results are
 * deterministic, and may differ in the last bits from an unsplit plan.
 *
 * sgemm_f32_ex_plan: the plan sgemm_f32_ex would run, host only, no HIP call:
 * *variant (an sgemm_f32_variant_id; 0 when no GEMM kernel runs), and for MFMA
 * variants *config, *group_m and *splits (the split count after rounding each
 * split's K extent up to a multiple of 32).  Returns 0, a positional error for
 * negative sizes, SGEMM_F32_ERR_TRANS, or SGEMM_F32_ERR_CONFIG for a NULL
 * output pointer.
 *
 * sgemm_f32_ex_config: runs one MFMA configuration with the given grouping
 * (1..64 tile rows) and requested split count (1..64; K is cut into extents
 * that are multiples of 32, so fewer splits may run).  Configurations 2-6 need
 * the 16-byte-load conditions of SGEMM_F32_MFMA_LARGE and return
 * SGEMM_F32_ERR_NOT_APPLICABLE otherwise; 0 and 1 fall back to 4-byte loads.
 * Configuration 6 stages 64 values of k per slice, so it also needs 64 stored
 * rows of each operand to span less than 2 GiB (SGEMM_F32_ERR_NOT_APPLICABLE
 * otherwise; the automatic choice then keeps its default plan).
 *
 * Configuration 5 is persistent and tile-scheduled: as many work-groups as fit
 * on the device at once take whole tiles in rounds, then equal shares of the
 * K slices of the tiles left over, so the last round is not left partly idle
 * (wave quantization, "Writing a Fast Matmul in CUDA, Step by Step", section
 * "Size effects"); tiles shared by several work-groups are summed in K order
 * by a second kernel.  It takes no split count (splits must be 1) and uses
 * the call's scratch (2 * 128 * 128 floats per resident work-group, 64 MiB
 * on MI355X) when tiles are shared.
 * Configuration 7 computes 256 x 256 tiles, one work-group per compute unit,
 * with the operands copied from memory straight into LDS.  It needs K, M of A
 * given transposed and N of B as given multiples of 4 (M of A as given and N
 * of B given transposed may be anything), the 16-byte-load conditions, 256 stored rows of an operand
 * read along k (16 of one read along M or N) spanning less than 2 GiB, and 256
 * rows of C spanning less than 2 GiB; SGEMM_F32_ERR_NOT_APPLICABLE otherwise.
 * It takes no split count (splits must be 1) and ignores the grouping.  The
 * automatic choice takes it when the plan would otherwise be the 128 x 128
 * grid without a split, the 256 x 256 grid has at least 256 tiles, and the
 * part of its rounds (256 tiles each) that lies inside C is at least 93 % and
 * within 2 % of the 128 x 128 grid's (a C stride too wide for it at call time
 * keeps the 128 x 128 grid).
 * Configurations 8, 9 and 10 run the kernel of configuration 7 on 128 x 128,
 * 64 x 64 and 192 x 192 tiles (two, four and one work-groups per compute unit)
 * with the same conditions; they honour the grouping and take no split count
 * (splits must be 1).  The automatic choice takes configuration 8 in place of the 128 x 128
 * grid and 9 in place of configuration 4, each without a split, when those
 * conditions hold, for configuration 9 also at most 1024 tiles of 64 x 64
 * (edge tiles included) (again, a C stride too wide at call time keeps the plan's
 * register-staged kernel).  It takes configuration 10 in place of an unsplit
 * 128 x 128 or 64 x 64 plan when the 192 x 192 grid has 250 to 256 tiles (one
 * round), and in place of an unsplit 64 x 64 plan when it has whole rounds
 * (at most 6 tiles short of a multiple of 256), K being at least 1024 (a C
 * stride too wide keeps the 128 x 128 grid).  A configuration 9 grid that spreads unevenly over the compute units
 * (the busiest holds at least 1.2 times the mean number of tiles) with K of
 * at least 1536 goes back to configuration 4 with K split in 2 or 3, and one
 * that is also one round of 250 to 256 tiles of 128 x 128 with K of at least
 * 1024 goes to configuration 8.
 * Where the automatic choice first copies misaligned operands to aligned
 * rows (SGEMM_F32_MFMA_SCALAR above), sgemm_f32_ex_plan reports the plan that
 * then runs on the copies; sgemm_f32_ex_config with that plan on the original
 * operands returns SGEMM_F32_ERR_NOT_APPLICABLE where it needs 16-byte loads.
 * A split plan whose partials exceed 1 GiB returns SGEMM_F32_ERR_TOO_LARGE.
 * Other arguments and return codes are those of sgemm_f32_ex.
 */
int sgemm_f32_ex_plan(int trans_a, int trans_b, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      int *variant, int *config, int *group_m, int *splits);

int sgemm_f32_ex_config(int config, int group_m, int splits, int trans_a, int trans_b,
                        int M, int N, int K, float alpha, const float *A, int lda,
                        const float *B, int ldb, float beta, float *C, int ldc,
                        hipStream_t stream);

/* Short static name of a configuration ("128x128", ...), or NULL if unknown. */
const char *sgemm_f32_config_name(int config);

/* 1 when a measured tuning table is compiled in, 0 when every shape uses the
   default choice. */
int sgemm_f32_tuning_table_present(void);

/* Short static name of a variant ("mfma_large", ...), or NULL if unknown. */
const char *sgemm_f32_variant_name(int variant);

/* Library version, e.g. 300 for 0.3.0. */
int sgemm_f32_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_H */
