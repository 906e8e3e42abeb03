/*
 * pdgemm.h -- multi-precision dense GEMM for AMD Instinct MI355X (gfx950).
 *
 * C = A * B in three precisions, each a hand-written HIP kernel on the
 * gfx950 matrix cores (MFMA):
 *
 *   gemm_f16  binary16 A, B -> fp32 accumulate -> fp32 C
 *   gemm_i8   int8 A, B     -> int32 accumulate -> int32 C
 *   gemm_i4   packed signed 4-bit A, B -> int32 accumulate -> int32 C
 *
 * The operation is the one studied in "Hand-Written PTX Tensor-Core GEMM
 * Kernels: A Multi-Precision Study on NVIDIA L4": GEMM in FP16, INT8 and INT4
 * (abstract; Section I), D = AB + C on the matrix units (Section II-A) taken
 * here with C = 0, and INT32 results without dequantization or scaling
 * (Section VI).  The operand roles follow the ".row.col" form of the MMA in
 * that paper's Listing 2: A is read along rows and B along columns, both
 * contiguous in K, which is also the "non-transposed B" layout that its
 * Section IV-D ablation finds fastest.
 *
 * ---------------------------------------------------------------------------
 * Layout (all three entry points)
 *   A   M x K, row-major:    element (i, k) at A[i*lda + k],  lda >= K
 *   B   K x N, column-major: element (k, j) at B[j*ldb + k],  ldb >= K
 *   C   M x N, row-major:    element (i, j) at C[i*ldc + j],  ldc >= N
 * The pages do not fix C's layout; row-major is the reading taken.
 *
 * gemm_i4: K, lda and ldb count 4-bit elements and must be even.  Element k
 * of a row sits in byte k/2 of that row (byte stride lda/2), in the low
 * nibble when k is even and the high nibble when k is odd, as a two's
 * complement value in [-8, 7].  The paper's INT4 type is signed (".s4",
 * Listing 2); the nibble order is not given there and low-nibble-first is the
 * reading taken.
 *
 * Semantics: C is overwritten with A*B (no alpha/beta).  K = 0 stores zeros
 * into the M x N block of C.  M = 0 or N = 0 is a no-op that returns 0.
 * Integer results are exact.  The exact sum must fit in int32 (always true
 * for K <= 131071); gemm_i4 additionally requires K <= 131071.  FP16 results
 * carry fp32 rounding only: every element satisfies
 * |C - sum_k a_ik b_kj| <= 1e-3 * sum_k |a_ik b_kj| for K up to 16384 (the
 * worst-case bound of K fp32 additions, K * 2^-24, stays below 1e-3).
 * Each FP16 sum runs in a fixed order, so a call gives the same bits every
 * time for a given shape and tile configuration.  The configurations without
 * a K split share one order and give the same bits as each other (the
 * 256 x 256 tile with column-major B runs 16 x 16 MFMAs, whose FP16 sums were
 * measured to round as those of the 32 x 32 ones, bit for bit); the K-split
 * configurations group K differently.  Where K is split across workgroups
 * (pdgemm_pick_splits below), FP16 takes two ranges whose binary32 partial
 * sums are added atomically into a zeroed C: 0 + x + y and 0 + y + x round
 * alike, so the bits still do not depend on which range finishes first.
 *
 * Alignment (checked): A and B 16-byte aligned, with lda and ldb spanning a
 * multiple of 16 bytes (f16: lda, ldb % 8 == 0; i8: % 16; i4: % 32); C
 * 4-byte aligned with any ldc >= N.  A row of A, B or C (lda, ldb, ldc
 * elements) may span at most 4 MiB.  M, N and K are otherwise arbitrary:
 * partial tiles are masked inside the kernels.  Operands are read in
 * 16-byte chunks: the chunk that holds the last element of a row may be read
 * whole (it never crosses the 16-byte granule of the allocation, since bases
 * and row spans are multiples of 16), and values outside the M x K and
 * K x N extents never reach a stored result.
 *
 * Ownership and execution: every pointer is device memory owned by the
 * caller, on the device the stream belongs to.  C must not overlap A, B or
 * the scales (the result is then undefined).  Where K is split across
 * workgroups, C is first zeroed and then receives the partial sums as
 * device-scope atomic adds, so it must be memory that supports them
 * (ordinary device allocations do).  The library never allocates,
 * frees, copies or synchronizes.  The call enqueues work on `stream` (a
 * hipStream_t passed as void*; NULL is the default stream) and returns once
 * it is enqueued.  Entry points are thread-safe and keep no state between
 * calls.
 *
 * Errors.  The convention follows "Chapter 5 · The Toolchain", Section 5.3
 * "Error handling that actually works" (the GPU programming book's toolchain
 * chapter): every call that can fail reports it, and because a launch is
 * asynchronous, a fault inside a kernel only shows at a later synchronizing
 * call, so catching it at its source takes a check after the launch plus a
 * synchronize, which serializes and is kept out of release and timing paths.
 * Here:
 *   - 0 on success;
 *   - negative values (PDGEMM_E* below) are argument errors, found on the
 *     host before any HIP call is made, with nothing enqueued;
 *   - positive values are hipError_t codes of the launch itself (the
 *     launch-time check of that section);
 *   - with the environment variable PDGEMM_SYNC_CHECK set to 1 at the first
 *     call, every call also synchronizes its stream and returns any execution
 *     error (the section's debug-build synchronize; off by default, since it
 *     serializes the caller's stream);
 *   - pdgemm_strerror() turns any of these codes into a message.
 * That section's checking macro prints and exits the process; a library must
 * not, so this one only returns codes and never aborts or exits.
 * ---------------------------------------------------------------------------
 */
#ifndef PDGEMM_H
#define PDGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes (error convention: "Chapter 5 · The Toolchain", Section 5.3;
 * see the file header). */
#define PDGEMM_OK 0
#define PDGEMM_EINVAL_DIM (-1)  /* M, N or K negative or too large (K > 2^30, over 2^32 work-items), or gemm_i4 K > 131071 */
#define PDGEMM_EINVAL_LD (-2)   /* lda < K, ldb < K (row-major B: ldb < N), ldc < N, or a row above 4 MiB */
#define PDGEMM_ENULL (-3)       /* NULL pointer for an operand with nonzero extent */
#define PDGEMM_EINVAL_I4 (-4)   /* gemm_i4: K, lda or ldb odd */
#define PDGEMM_EALIGN (-5)      /* a pointer or leading dimension breaks the alignment rules */
#define PDGEMM_EINVAL_CFG (-6)  /* unknown precision or tile configuration, or a dequantizing
                                   epilogue for FP16; reported before any other check.  Every
                                   configuration, the K-split ones included, serves both B layouts */

#define PDGEMM_EWORKSPACE (-7)  /* a workspace or FP6 image smaller than its entry point needs
                                   (pdgemm_i4_workspace_size(), pdgemm_i4_f6_image_bytes()),
                                   a negative size, or one not 16-byte aligned */

#define PDGEMM_I4_MAX_K 131071

/* FP16 inputs (IEEE binary16 bit patterns), fp32 accumulation, fp32 output. */
int gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
             const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream);

/* INT8 inputs, int32 accumulation, int32 output. */
int gemm_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
            const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);

/* Packed signed INT4 inputs (two per byte along K, even k in the low nibble),
 * int32 accumulation, int32 output.  K, lda, ldb count 4-bit elements. */
int gemm_i4(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
            const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);

/* INT8 / INT4 GEMM followed by a dequantizing epilogue.
 *
 * The paper ("Hand-Written PTX Tensor-Core GEMM Kernels ...", Section VI)
 * stops at the INT32 sums and leaves dequantization out; this is the step an
 * inference pipeline applies next.  With S the exact integer sum of gemm_i8 /
 * gemm_i4,
 *     C[i][j] = ((float)S[i][j] * scale_a[i]) * scale_b[j]
 * evaluated in IEEE binary32 in that order (each step rounded to nearest
 * even), then stored as binary32 (out_f16 = 0; C is float*) or rounded once
 * more to binary16 (out_f16 = 1; C holds binary16 bit patterns, overflow
 * gives infinity).  The result is unique, so it is reproducible bit for bit.
 * scale_a holds M floats (one per row of A), scale_b N floats (one per
 * column of B), both 4-byte aligned device memory owned by the caller and
 * only read.  K = 0 gives (0 * scale_a[i]) * scale_b[j] (a signed zero, or
 * NaN for an infinite scale).  C is 4-byte aligned for binary32 output and
 * 2-byte aligned for binary16; ldc counts output elements.  Other arguments,
 * layouts and errors as gemm_i8 / gemm_i4; a null scale pointer with
 * M, N > 0 returns PDGEMM_ENULL. */
int gemm_i8_dequant(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                    const int8_t *B, int64_t ldb, const float *scale_a, const float *scale_b,
                    void *C, int64_t ldc, int out_f16, void *stream);
int gemm_i4_dequant(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                    const uint8_t *B, int64_t ldb, const float *scale_a, const float *scale_b,
                    void *C, int64_t ldc, int out_f16, void *stream);

/* C = A * B with B row-major (N-contiguous): element (k, j) of B at
 * B[k*ldb + j] with ldb >= N.  This is the "transposed B" layout of the
 * paper's loader ablation (Section IV-D, Run 4), which it finds slower than
 * the column-major B of the entry points above; here the kernels read it with
 * gfx950's transposing LDS loads, so both layouts feed the same MFMAs.
 * gemm_i4_rowb: B packs two signed 4-bit values per byte along N (element j
 * of a row in byte j/2, low nibble for even j); ldb counts 4-bit elements and
 * must be even, K must be even (A's packing), N may be odd.  Other
 * arguments, alignment (ldb spans a multiple of 16 bytes), results and
 * errors as gemm_f16 / gemm_i8 / gemm_i4, with ldb < N giving
 * PDGEMM_EINVAL_LD. */
int gemm_f16_rowb(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                  const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream);
int gemm_i8_rowb(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                 const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);
int gemm_i4_rowb(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                 const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);

/* INT4 GEMM on the FP6 matrix cores, with a caller-provided workspace.
 *
 * The same operation, layouts, results (bit for bit) and errors as gemm_i4,
 * gemm_i4_rowb and gemm_i4_dequant.  gfx950 has no signed 4-bit MFMA; the
 * entry points above run INT4 on the INT8 MFMA as two nibble planes, two
 * MFMAs per 64 values of K.  These run it on the FP6 MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4, about twice the INT8 MFMA rate), one
 * MFMA per 64 values: every INT4 value v is exact as the e2m3 value v / 8,
 * block scales of 2^3 on both operands make each product the integer a * b,
 * and the fp32 accumulators hold exact integers (|C| <= 64 K < 2^24).  A
 * pre-pass converts A and B into that format once, into the workspace
 * (3/4 of a byte per value, in 32-row x 128-value units; B row-major is
 * transposed there), and the GEMM reads the workspace.  This replaces the
 * paper's native m16n8k64 .s4 MMA ("Hand-Written PTX Tensor-Core GEMM
 * Kernels ...", Listing 2, Section IV-C), which has no gfx950 counterpart.
 *
 * pdgemm_i4_workspace_size() gives the bytes a shape needs, or 0 where the
 * entry points run the INT8-MFMA kernels instead (shapes of few tiles, where
 * the pre-pass would not pay; the workspace may then be NULL).  The
 * workspace is device memory owned by the caller, 16-byte aligned, not
 * overlapping A, B, C or the scales; its contents on return are undefined.
 * Calls that share a workspace must not run concurrently.  Both kernels are
 * enqueued on `stream`; nothing is allocated or synchronized.  A workspace
 * that is NULL (with a nonzero size needed) returns PDGEMM_ENULL, one that
 * is too small or misaligned PDGEMM_EWORKSPACE. */
int64_t pdgemm_i4_workspace_size(int64_t M, int64_t N, int64_t K);
int gemm_i4_ws(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
               const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc,
               void *workspace, int64_t workspace_bytes, void *stream);
int gemm_i4_rowb_ws(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                    const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc,
                    void *workspace, int64_t workspace_bytes, void *stream);
int gemm_i4_dequant_ws(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                       const uint8_t *B, int64_t ldb, const float *scale_a,
                       const float *scale_b, void *C, int64_t ldc, int out_f16,
                       void *workspace, int64_t workspace_bytes, void *stream);

/* The FP6 path with an explicit tile configuration (0 <= cfg <
 * pdgemm_i4_f6_num_configs()), whatever the shape: B column-major or (with
 * b_rowmajor) row-major; with scale_a and scale_b non-NULL the dequantizing
 * epilogue (C fp32, or binary16 with out_f16), else int32 C.  The workspace
 * must hold what pdgemm_i4_f6_workspace_bytes() gives.  pdgemm_i4_f6_pick()
 * is the configuration the *_ws entry points take for a shape (-1: the
 * INT8-MFMA kernels). */
int pdgemm_i4_f6_cfg(int cfg, int b_rowmajor, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, const void *B, int64_t ldb,
                     const float *scale_a, const float *scale_b, void *C, int64_t ldc,
                     int out_f16, void *workspace, int64_t workspace_bytes, void *stream);
int pdgemm_i4_f6_num_configs(void);
int pdgemm_i4_f6_pick(int64_t M, int64_t N, int64_t K);
int64_t pdgemm_i4_f6_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* INT4 with B converted once: the FP6 route for a B that serves many calls
 * (the weights of an inference layer, say), so that a call converts only A.
 *
 * pdgemm_i4_f6_pack() converts one INT4 operand into its FP6 image (the
 * format the *_ws entry points build in their workspace; 3/4 of a byte per
 * value, pdgemm_i4_f6_image_bytes(rows, K) bytes): `rows` rows of K values
 * packed along K (a column-major B given as its N rows, i.e. Bt; src_rowmajor
 * = 0), or a row-major B, K rows of `rows` values packed along the row
 * (src_rowmajor = 1).  ld counts 4-bit elements as in gemm_i4 / gemm_i4_rowb
 * and the same alignment rules hold.  The image is device memory owned by the
 * caller, 16-byte aligned; it depends only on the operand's values and K.
 *
 * gemm_i4_packed_b() computes the same C as gemm_i4 (bit for bit) from A and
 * the image of B, which must have been packed from N rows of B with the same
 * K.  A's image is built in the workspace (pdgemm_i4_f6_image_bytes(M, K)
 * bytes, 16-byte aligned, caller-owned; contents undefined on return).  B's
 * image is only read, so calls may share it; calls sharing a workspace must
 * not overlap.  gemm_i4_dequant_packed_b() is the dequantizing form (as
 * gemm_i4_dequant), pdgemm_i4_packed_b_cfg() takes an explicit FP6 tile
 * configuration (0 <= cfg < pdgemm_i4_f6_num_configs(); with scale_a and
 * scale_b non-NULL the dequantizing epilogue).  Both kernels are enqueued on
 * `stream`; nothing is allocated or synchronized.  Errors as gemm_i4; an
 * image or workspace that is too small or misaligned returns
 * PDGEMM_EWORKSPACE, a NULL one PDGEMM_ENULL. */
int64_t pdgemm_i4_f6_image_bytes(int64_t rows, int64_t K);
int pdgemm_i4_f6_pack(int64_t rows, int64_t K, const uint8_t *src, int64_t ld, int src_rowmajor,
                      void *image, int64_t image_bytes, void *stream);
int gemm_i4_packed_b(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                     const void *image_b, int64_t image_b_bytes, int32_t *C, int64_t ldc,
                     void *workspace, int64_t workspace_bytes, void *stream);
int gemm_i4_dequant_packed_b(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                             const void *image_b, int64_t image_b_bytes, const float *scale_a,
                             const float *scale_b, void *C, int64_t ldc, int out_f16,
                             void *workspace, int64_t workspace_bytes, void *stream);
int pdgemm_i4_packed_b_cfg(int cfg, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                           const void *image_b, int64_t image_b_bytes, const float *scale_a,
                           const float *scale_b, void *C, int64_t ldc, int out_f16,
                           void *workspace, int64_t workspace_bytes, void *stream);

/* gemm_i4 for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * It is gemm_i4_ws with the workspace taken from a fixed file-scope device
 * array of pdgemm_i4_noalloc_max_bytes() bytes (128 MiB, enough for
 * M = N = K = 8192), of which each GPU the library runs on holds one copy
 * until the process ends; nothing is allocated or freed by the call.
 * Shapes that the workspace entry points run on the INT8-MFMA kernels do not
 * touch the array.  A shape whose FP6 workspace would exceed the array
 * returns PDGEMM_EWORKSPACE, before any launch.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress) and may return its hipError_t; devices with an index
 * of 64 or more return hipErrorInvalidDevice.  Arguments, results and other
 * errors as gemm_i4. */
int gemm_i4_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                    const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);
int64_t pdgemm_i4_noalloc_max_bytes(void);

/* Precision ids and tile configurations, for the calls below. */
#define PDGEMM_PREC_F16 0
#define PDGEMM_PREC_I8 1
#define PDGEMM_PREC_I4 2

/* The same GEMM with an explicit tile configuration (0 <= cfg <
 * pdgemm_num_configs()); the three entry points above pick one by shape.
 * Same arguments, layout, alignment and error rules; A, B, C are passed as
 * untyped device pointers of the precision's element type. */
int pdgemm_gemm_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda, const void *B, int64_t ldb,
                    void *C, int64_t ldc, void *stream);

/* The row-major-B GEMM with an explicit tile configuration. */
int pdgemm_gemm_rowb_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A,
                         int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                         void *stream);

/* K split across workgroups.  The entry points that return raw sums
 * (gemm_f16, gemm_i8, gemm_i4 and their _rowb, _ws and _noalloc forms, where
 * those run the INT8-MFMA kernels) split K into `splits` ranges when the
 * shape has too few tiles to fill the GPU and K is long: a kernel zeroes the
 * M x N block of C, then each range, a row of the launch grid, adds its
 * partial tile with atomic adds.  Integer results are exact in any order;
 * FP16 takes at most two ranges (see Semantics).  The pages describe no such
 * split; it serves the few-tile shapes whose small-N regime the paper studies
 * ("Hand-Written PTX Tensor-Core GEMM Kernels ...", Section IV, the 3-stage
 * INT4 kernel at small N).  The dequantizing entry points never split.
 *
 * pdgemm_pick_splits: the split the raw-sum entry points use for a shape and
 * B layout (b_rowmajor 0 or 1): returns the number of ranges (1 = no split,
 * -1 for an unknown precision) and stores the tile configuration in *cfg
 * (may be NULL).
 *
 * pdgemm_gemm_splitk_cfg: the GEMM with an explicit tile configuration and
 * split.  cfg must be one of the tiles a split runs on (2 or 5), splits >= 1;
 * K is cut into ranges of ceil(K / splits) values rounded up to a whole
 * 128-byte stage, so fewer ranges may result; for FP16 more than two ranges
 * give PDGEMM_EINVAL_CFG.  splits == 1 or K == 0 runs the plain kernel of cfg.
 * Other arguments, layouts and errors as pdgemm_gemm_cfg (b_rowmajor 0) or
 * pdgemm_gemm_rowb_cfg (b_rowmajor 1). */
int pdgemm_pick_splits(int prec, int b_rowmajor, int64_t M, int64_t N, int64_t K, int *cfg);
int pdgemm_gemm_splitk_cfg(int prec, int cfg, int b_rowmajor, int splits, int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                           void *stream);

/* The dequantizing GEMM with an explicit tile configuration (prec is
 * PDGEMM_PREC_I8 or PDGEMM_PREC_I4; FP16 returns PDGEMM_EINVAL_CFG). */
int pdgemm_dequant_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A,
                       int64_t lda, const void *B, int64_t ldb, const float *scale_a,
                       const float *scale_b, void *C, int64_t ldc, int out_f16, void *stream);

/* Number of tile configurations, and the one the entry points pick for a
 * shape (-1 for an unknown precision) when they do not split K across
 * workgroups. */
int pdgemm_num_configs(void);
int pdgemm_pick_config(int prec, int64_t M, int64_t N, int64_t K);

/* Tile configuration cfg: block tile rows/cols, wave tile rows/cols,
 * workgroup size in threads.  Returns 0, or PDGEMM_EINVAL_CFG.  Any output
 * pointer may be NULL. */
int pdgemm_config_info(int cfg, int *block_m, int *block_n, int *wave_m, int *wave_n,
                       int *threads);

/* Static message for a return code (never NULL): the PDGEMM_E* codes above,
 * or hipGetErrorString() for a positive hipError_t.  Part of the error
 * convention of "Chapter 5 · The Toolchain", Section 5.3 (every error made
 * readable where it is reported). */
const char *pdgemm_strerror(int code);

/* Library version as major*10000 + minor*100 + patch.  No passage of the
 * pages defines a version query; it exists so that a caller can check which
 * build it loaded. */
int pdgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PDGEMM_H */
