/*
 * dense_gemm.h -- C ABI of the MI355X (gfx950) tiled dense GEMM library
 * (libdense_gemm.so).
 *
 * Operation.  "TIRx GEMM on Blackwell", section "The short version", defines
 * the product D = A @ B.T with FP16 inputs and output and FP32 accumulation.
 * TileFoundry "Choosing schedules and instructions for a backend", section 1
 * (the GRID HIR), defines D = a @ b with a (M, K) and b (K, N) in BF16: the
 * accumulator starts at zero in f32, every K block adds its partial product,
 * and the accumulator is cast to the output type once.  Section 6 of that
 * page adds that the output need not be cleared before each tile overwrites
 * it: D is overwritten, with no alpha, beta, bias or activation.
 *
 * Layout.  All matrices are row-major with an explicit leading dimension, as
 * in the conventional layout rule of the CMU TIRx blog ("Conventional
 * layouts": element (i, j) of a matrix with leading dimension ld sits at
 * offset i * ld + j elements):
 *   A  M x K, element (i, k) at A[i * lda + k]                  (lda >= K)
 *   B  "nt": N x K, element (j, k) at B[j * ldb + k]            (ldb >= K)
 *      "nn": K x N, element (k, j) at B[k * ldb + j]            (ldb >= N)
 *   D  M x N, element (i, j) at D[i * ldd + j]                  (ldd >= N)
 * Elements are 16-bit patterns (IEEE binary16 for *_f16, bfloat16 for
 * *_bf16) passed as untyped device pointers.  Results are rounded from the
 * FP32 accumulator to the output format with round-to-nearest-even.
 *
 * Semantics.  For 0 <= i < M, 0 <= j < N:
 *     D[i][j] = round( sum_{k < K} A[i][k] * Bhat[k][j] )
 * with the sum accumulated in FP32 in an order the library chooses (fixed per
 * tile configuration, so repeated calls are bitwise reproducible).  Elements
 * of D outside [0, M) x [0, N) -- including the columns between N and ldd --
 * are never written.  K == 0 writes zeros; M == 0 or N == 0 does nothing.
 *
 * Alignment.  A, B and D need only the 2-byte alignment of their elements
 * (an odd address returns DENSE_GEMM_MISALIGNED); M, N, K and the leading
 * dimensions are otherwise arbitrary (ragged edges are masked, and K need not
 * be a multiple of the tile depth).  The tiled kernel moves A and B in
 * 16-byte chunks: it reads an operand in place when its pointer is 16-byte
 * aligned and its leading dimension and row length (K; N for the "nn" B) are
 * multiples of 8 elements.  Any other operand is first copied by a repack
 * kernel into a dense, zero-padded copy in the workspace (one extra pass over
 * that operand; the result is the same).  D is written with 16-byte stores
 * where its rows are 16-byte aligned and element by element otherwise.
 *
 * Split-K.  When the tiles of the last, partial wave over the CUs (all
 * tiles, when there are fewer tiles than CUs) would leave CUs idle and K is
 * long enough for the parts to pay for their partial sums (see
 * dense_gemm_plan), the K dimension of those tiles is split: each part
 * writes an FP32 partial tile to the workspace and a second kernel sums them
 * in a fixed order (results stay reproducible) and rounds once.  The other
 * tiles are computed whole in the same launch.  dense_gemm_ex can force a
 * number of parts, or none (dense_gemm_options).
 *
 * Tile width and rows.  Output tiles are 256 x 256.  For D = A @ B.T they
 * are 256 x 128 instead when N <= 128 (one tile column either way, half the
 * work of a half-empty 256-wide tile), or when 256-wide tiles would occupy
 * at most half the CUs and the operands take at most 192 MiB (twice the
 * tiles, one wave).  Products with M <= 128 use tiles of 128 rows (one tile
 * row either way, half the work of a half-empty 256-row tile).  Every tile
 * shape sums each output in the same order, so unsplit results are
 * identical.  dense_gemm_ex can force the width of A @ B.T.
 *
 * Small outputs.  A product with M <= 128 and K <= 16384 whose 16 x 16
 * tiles number at most 512, or form a single tile row (M <= 16), or (A @
 * B.T) whose 32 x 32 tiles times K are at most 2^21, runs a second kernel
 * instead of the tiled one: one workgroup per tile of D (16 x 16; for
 * A @ B.T 32 x 16 or 32 x 32 where dense_gemm_plan gives them), whose eight
 * waves split K among themselves and add their FP32 sums in a fixed order
 * (reproducible, and the same bits whatever the tile shape; no workspace
 * unless an operand is repacked).  For D = A @ B it also needs K <= 4096
 * and at most 21 * 2^20 B elements streamed by its tiles, ceil(M / 16) * N
 * * K (its tiles read B in 32-byte row segments; past that the tiled
 * kernel is faster); A @ B and A @ B.T on the same operands then give the
 * same result bit for bit.
 * Its summation order differs from the tiled kernel's, within the same
 * rounding bound.  Any dense_gemm_options override asks for the tiled
 * kernel instead.
 *
 * Workspace.  A call that repacks an operand or splits K needs device
 * memory beyond A, B and D: dense_gemm_workspace_size gives the amount.
 * dense_gemm_ex takes it from the caller (the destination-passing form of
 * TileFoundry's schedule tutorial, section 6, whose lowered kernel takes its
 * scratch buffers as arguments) and allocates nothing.  The plain entry
 * points (gemm_nt_f16 and the rest, whose argument list has no workspace)
 * take it with hipMallocAsync on `stream` and return it with hipFreeAsync on
 * the same stream (stream-ordered, from the device's default memory pool);
 * if it cannot be had, a split call runs unsplit and a call that needs a
 * repack returns DENSE_GEMM_NO_MEMORY (nothing launched).  Aligned operands
 * with enough output tiles need none.
 *
 * Ownership and concurrency.  The caller owns every buffer and the stream.
 * The library keeps no pointers after a call returns and caches only
 * per-device properties (thread-safe); apart from the workspace above it
 * allocates no device memory.  A, B, D and a workspace must not overlap.
 * Calls are asynchronous and ordered on `stream` (0 is the null stream); the
 * caller synchronizes.  Calls on different streams may run concurrently (each
 * with its own workspace).
 *
 * Errors.  Every entry point validates its arguments before launching and
 * returns a dense_gemm_status; on any error nothing is launched and D is
 * untouched.  DENSE_GEMM_LAUNCH_FAILED reports an error from the HIP runtime
 * at launch time (asynchronous faults surface at the caller's next
 * synchronization, as for any HIP kernel).
 */
#ifndef DENSE_GEMM_H
#define DENSE_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle (identical to its own declaration). */
typedef struct ihipStream_t* hipStream_t;

typedef enum dense_gemm_status {
  DENSE_GEMM_OK = 0,
  DENSE_GEMM_INVALID_DIM = 1,   /* M, N or K negative */
  DENSE_GEMM_NULL_PTR = 2,      /* D null with M*N > 0; A or B null with M*N*K > 0 */
  DENSE_GEMM_BAD_LD = 3,        /* a leading dimension below its minimum */
  DENSE_GEMM_MISALIGNED = 4,    /* A, B or D at an odd address */
  DENSE_GEMM_TOO_LARGE = 5,     /* a dimension >= 2^31, 2^31 or more output tiles,
                                   or a per-tile operand span >= 2^31 bytes */
  DENSE_GEMM_LAUNCH_FAILED = 6, /* the HIP runtime rejected the launch */
  DENSE_GEMM_NO_DEVICE = 7,     /* no current HIP device, or it is not a gfx950 */
  DENSE_GEMM_BAD_ARG = 8,       /* an argument of a helper below is out of its range */
  DENSE_GEMM_NO_MEMORY = 9,     /* no device memory for the workspace */
  DENSE_GEMM_WORKSPACE_TOO_SMALL = 10, /* the caller's workspace is null or smaller
                                          than the size query reports */
  DENSE_GEMM_SCRATCH_TOO_SMALL = 11    /* gemm_nt_f16_noalloc: the call needs more than
                                          its fixed 64 MiB of scratch */
} dense_gemm_status;

/* The four type and layout pairings, for dense_gemm_ex and
 * dense_gemm_workspace_size. */
typedef enum dense_gemm_op {
  DENSE_GEMM_NT_F16 = 0,   /* D = A @ B.T, FP16 (gemm_nt_f16)  */
  DENSE_GEMM_NN_BF16 = 1,  /* D = A @ B,   BF16 (gemm_nn_bf16) */
  DENSE_GEMM_NT_BF16 = 2,  /* D = A @ B.T, BF16 (gemm_nt_bf16) */
  DENSE_GEMM_NN_F16 = 3    /* D = A @ B,   FP16 (gemm_nn_f16)  */
} dense_gemm_op;

/* Overrides of the library's launch plan (a null pointer, or zeros, keep
 * its own choice).  They change the FP32 summation order of the outputs they
 * touch (split_k), or the tiling (tile_n, which keeps the order), never the
 * operation; both stay within the rounding bound.  Either one, non-zero,
 * selects the tiled kernel (not the small-output kernel).
 *   split_k  0: the library's choice; 1: no split; n > 1: every tile's K
 *            steps in min(n, steps) parts of equal length (the last shorter)
 *   tile_n   0: the library's choice; 256; or 128 (D = A @ B.T only).  A
 *            width other than the library's own drops its split-K choice
 *            (made for its width): split_k 0 then means no split.
 * A forced split whose partial tiles would exceed 2^62 bytes of workspace
 * returns DENSE_GEMM_TOO_LARGE. */
typedef struct dense_gemm_options {
  int32_t split_k;
  int32_t tile_n;
} dense_gemm_options;

/* D = A @ B.T; FP16 in, FP32 accumulate, FP16 out.  A is M x K, B is N x K.
 * The FP16 product of "TIRx GEMM on Blackwell", "The short version". */
dense_gemm_status gemm_nt_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                              const void* B, int64_t ldb, void* D, int64_t ldd,
                              hipStream_t stream);

/* D = A @ B; BF16 in, FP32 accumulate, BF16 out.  A is M x K, B is K x N.
 * The BF16 product of TileFoundry's schedule tutorial, section 1. */
dense_gemm_status gemm_nn_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                               const void* B, int64_t ldb, void* D, int64_t ldd,
                               hipStream_t stream);

/* The other two combinations of the same operation (same kernels, other
 * template arguments): D = A @ B.T in BF16 and D = A @ B in FP16. */
dense_gemm_status gemm_nt_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                               const void* B, int64_t ldb, void* D, int64_t ldd,
                               hipStream_t stream);
dense_gemm_status gemm_nn_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                              const void* B, int64_t ldb, void* D, int64_t ldd,
                              hipStream_t stream);

/* The optimisation steps of "TIRx GEMM on Blackwell" (sections V3 to V9)
 * rebuilt one idea at a time, for measurement: D = A @ B.T in FP16 as
 * gemm_nt_f16 computes it, by the kernel of `level`:
 *   1  one 128 x 128 tile per workgroup, threads copy A and B into LDS, then
 *      compute (no overlap)                                       (V3)
 *   2  as 1, the tiles moved by LDS-DMA loads                      (V4)
 *   3  as 2, two LDS stages (loads of step k+1 overlap step k)     (V5)
 *   4  as 3, persistent workgroups in the grouped XCD-aware order  (V6)
 *   5  as 4, 256 x 256 tiles (each staged tile feeds two waves)    (V8/V9)
 *   6  gemm_nt_f16 itself
 *   7  as 4, with a fifth wave that issues every load while four
 *      waves compute (warp specialization)                        (V7)
 *   8  as 5, with v_mfma_f32_32x32x16 in place of the 16 x 16 x 32
 *      MFMA (a comparison of the two MFMA shapes, not a page step)
 *   9  as 5, with eight waves of 128 x 64 (two per SIMD) in place of
 *      four of 128 x 128 (a comparison, not a page step)
 * Levels 1-5 and 7-9 take only shapes that divide their tile: M and N
 * multiples of 128 (256 for levels 5, 8 and 9), K a positive multiple of
 * 64, A, B and D 16-byte aligned with lda, ldb and ldd multiples of 8
 * (DENSE_GEMM_BAD_ARG, _BAD_LD, _MISALIGNED or _TOO_LARGE otherwise; a
 * level outside 1..9 is DENSE_GEMM_BAD_ARG).  Same ownership, stream and error rules as the
 * entry points above; the FP32 accumulation order differs between levels,
 * so results agree within the rounding bound, not bit for bit. */
dense_gemm_status gemm_nt_f16_ladder(int level, int64_t M, int64_t N, int64_t K, const void* A,
                                     int64_t lda, const void* B, int64_t ldb, void* D,
                                     int64_t ldd, hipStream_t stream);

/* FP8 block-scaled product: D = A @ B.T with E4M3 elements and one E8M0
 * scale per 32 consecutive K values of each row, FP32 accumulation, BF16 out.
 * The CMU TIRx blog ("Evaluation", "Kernel performance") benchmarks an FP8
 * block-scaled GEMM without fixing its encodings; this entry point takes the
 * OCP microscaling (MX) reading, the format gfx950's scaled MFMA applies:
 *     D[i][j] = round_bf16( sum_{k < K} SA[i][k/32] A[i][k] * SB[j][k/32] B[j][k] )
 * where A[i][k], B[j][k] are the E4M3 ("fn": no infinities, S.1111.111 is
 * NaN, largest 448) values of the byte codes and SA, SB the E8M0 scales
 * 2^(code - 127) (code 255 is NaN).  Both operands are K-major:
 *   A   M x K bytes, element (i, k) at A[i * lda + k]
 *   B   N x K bytes, element (j, k) at B[j * ldb + k]
 *   SA  M x K/32 bytes, scale of block b of row i at SA[i * ldsa + b]
 *   SB  N x K/32 bytes, scale of block b of row j at SB[j * ldsb + b]
 *   D   M x N bfloat16, element (i, j) at D[i * ldd + j]
 * K must be a multiple of 32 (DENSE_GEMM_BAD_ARG otherwise); A and B must be
 * 16-byte aligned with lda and ldb multiples of 16 (DENSE_GEMM_MISALIGNED);
 * D needs 2-byte alignment.  M, N and K/128 may be ragged.  The products are
 * exact in FP32; their sum is accumulated in FP32 in a fixed order (results
 * are reproducible on a device; the order depends on the plan, hence on the
 * CU count).  Small outputs (M <= 128, K <= 8192, and M <= 16, or at most
 * 1024 tiles of 32 x 32 in D, or at most 1536 with tiles * K <= 2^23) run a
 * small-output kernel (tiles of 16 x 16, 32 x 16 or 32 x 32 as
 * gemm_nt_e4m3_mx_plan gives, K split among eight waves, the scales staged
 * in LDS; every tile shape gives the same bits) that needs no workspace.
 * Other products run a tiled kernel (256 x 256 tiles) that takes a
 * workspace (hipMallocAsync / hipFreeAsync on `stream`;
 * DENSE_GEMM_NO_MEMORY if unavailable) of 1 KiB per 256-row tile of A and
 * of B per 128 K values for the repacked scales, plus, where the plan
 * splits K (gemm_nt_e4m3_mx_plan: the tiles of a last, partial wave, or all
 * tiles when there are fewer than CUs), 256 KiB per part of each split tile
 * for its FP32 partial sums, which a second kernel adds in part order and
 * rounds to BF16.  The other rules (zeros for K == 0, ownership, stream
 * order, errors) are those stated at the top of this file. */
dense_gemm_status gemm_nt_e4m3_mx(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                  const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                  const void* SB, int64_t ldsb, void* D, int64_t ldd,
                                  hipStream_t stream);

/* ---- caller-owned workspace (nothing allocated) ------------------------
 * The workspace-passing forms of the entry points above, for callers that
 * manage device memory themselves (a memory pool, graph capture, a serving
 * loop): the same operation, kernels and results (bit for bit, for the same
 * options), with the scratch memory given as `workspace` (256-byte aligned,
 * at least the size the query reports; it may be null when that size is
 * 0).  A workspace below the size returns DENSE_GEMM_WORKSPACE_TOO_SMALL,
 * one off 256-byte alignment DENSE_GEMM_MISALIGNED, before any launch.  The
 * workspace is used by the launches of this call only (stream-ordered:
 * after the call's work on `stream` completes it may be reused; two calls in
 * flight at once need two workspaces).  Its contents need no initialisation
 * and are left undefined. */

/* Bytes of workspace dense_gemm_ex needs for these arguments (0 if none).
 * `op` is a dense_gemm_op; the pointers A and B are only tested for null
 * and alignment (an operand off 16-byte alignment, or with K, its leading
 * dimension or, for the A @ B layout's B, N not a multiple of 8, takes a
 * repacked copy).  num_cus: the device's compute units (0: query the
 * current device).  `opt` as for dense_gemm_ex (may be null).  Errors as
 * dense_gemm_validate, DENSE_GEMM_BAD_ARG for a bad op, option or null
 * `bytes`, DENSE_GEMM_NO_DEVICE if num_cus is 0 and no gfx950 is current. */
dense_gemm_status dense_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K,
                                            const void* A, int64_t lda, const void* B,
                                            int64_t ldb, int64_t num_cus,
                                            const dense_gemm_options* opt, size_t* bytes);

/* The product `op` (a dense_gemm_op) with the caller's workspace and
 * optional plan overrides; arguments, layouts and errors as the entry point
 * of that op. */
dense_gemm_status dense_gemm_ex(int op, int64_t M, int64_t N, int64_t K, const void* A,
                                int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd,
                                const dense_gemm_options* opt, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* gemm_nt_f16 for callers that cannot allocate device memory at all (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc) and keep no workspace of their own: the same arguments, plan,
 * kernels and results (bit for bit), with the scratch memory taken from a
 * fixed 64 MiB array that the library holds on each device it runs on from
 * its first use until the process ends.  A call that needs more (repacked
 * operands beyond it; every split-K plan on a 256-CU device fits) returns
 * DENSE_GEMM_SCRATCH_TOO_SMALL before any launch.  It calls no allocator.
 * All calls on one device share that array and leave their contents in it:
 * two calls whose work overlaps on one device (on different streams, or
 * from different threads) race and give undefined results; calls ordered
 * on one stream, or synchronized, are safe.  Nothing in it needs to start
 * at zero. */
dense_gemm_status gemm_nt_f16_noalloc(int64_t M, int64_t N, int64_t K, const void* A,
                                      int64_t lda, const void* B, int64_t ldb, void* D,
                                      int64_t ldd, hipStream_t stream);

/* Bytes of workspace gemm_nt_e4m3_mx_ex needs on a device with num_cus
 * compute units (0: query the current device): the repacked scale panels,
 * 1 KiB per 256-row tile of A and of B per 128 K values, and the FP32
 * partial tiles of a split-K plan, 256 KiB per part of each split tile (0
 * when M or N is 0, and for the small-output kernel).  DENSE_GEMM_BAD_ARG
 * for K not a multiple of 32, a negative num_cus or a null `bytes`,
 * DENSE_GEMM_NO_DEVICE if num_cus is 0 and no gfx950 is current. */
dense_gemm_status gemm_nt_e4m3_mx_workspace_size(int64_t M, int64_t N, int64_t K,
                                                  int64_t num_cus, size_t* bytes);

/* gemm_nt_e4m3_mx with the caller's workspace. */
dense_gemm_status gemm_nt_e4m3_mx_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                     const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                     const void* SB, int64_t ldsb, void* D, int64_t ldd,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* A static, human-readable name for a status code (never NULL). */
const char* dense_gemm_status_string(int status);

/* ---- host-only helpers (no device call; usable without a GPU) ---------- */

/* The argument check every entry point runs first.  layout: 0 = "nt",
 * 1 = "nn".  Pointers are only compared with NULL and tested for alignment. */
dense_gemm_status dense_gemm_validate(int layout, int64_t M, int64_t N, int64_t K,
                                      const void* A, int64_t lda, const void* B, int64_t ldb,
                                      const void* D, int64_t ldd);

/* The persistent tile scheduler's map from a workgroup's task index to the
 * output tile it computes: tiles are visited in groups of group_m tile rows,
 * column by column within a group (the grouped traversal of TileFoundry's
 * schedule tutorial, section 3), the last group possibly shorter.  Writes the
 * tile row and column.  Returns DENSE_GEMM_BAD_ARG if task is outside
 * [0, tiles_m * tiles_n) or a size is not positive. */
dense_gemm_status dense_gemm_tile_of_task(int64_t task, int64_t tiles_m, int64_t tiles_n,
                                          int64_t group_m, int64_t* tile_m, int64_t* tile_n);

/* The launch plan for a problem on a device with num_cus compute units.
 * Writes 10 values to out: the tile rows BM (256, or 128 when M <= 128),
 * the tile width BN (256, or 128 as described under "Tile width and rows"
 * above), BK, tiles_m, tiles_n, grid (workgroups of the
 * GEMM kernel), group_m, threads per workgroup, the number of K splits
 * (1: none) and the K steps (of BK) per split.  For the small-output kernel
 * ("Small outputs" above) the grid is tiles_m * tiles_n workgroups of 512
 * threads, group_m 1 and no split; its tiles are 16 x 16 for A @ B and for
 * M <= 16, else 32 x 32 where those number at least num_cus, else 32 x 16
 * where those do, else 16 x 16.  Split-K applies to the
 * r = tiles mod num_cus tiles of the last, partial wave (all tiles when
 * tiles < num_cus), with K spanning at least 8 steps, at most one part per
 * CU (r * parts <= num_cus) and at least 4 steps per part.  When tiles <
 * num_cus the number of parts p minimises the estimate (in 0.01 us)
 * ceil(steps / p) * 105 + 1200 + 12 * f * p * r against steps * 105
 * unsplit, for 256-wide tiles (70 and 6 for 128-wide ones), with f the
 * share of a tile's 16-row blocks inside D (ceil(M / 16) / 16 when M < 256,
 * else 1: partial tiles skip the blocks outside D) -- a model fitted to
 * times measured on the MI355X; when tiles > num_cus the last wave is
 * split, into as many parts as fit, only if 4 r <= num_cus.  The grid is
 * then r * parts when tiles < num_cus, else num_cus. */
dense_gemm_status dense_gemm_plan(int layout, int64_t M, int64_t N, int64_t K,
                                  int64_t num_cus, int64_t* out);

/* The launch plan of gemm_nt_e4m3_mx for M, N > 0 and K a multiple of 32
 * on a device with num_cus compute units, as 10 values in the format of
 * dense_gemm_plan: tile rows and columns, the K depth of a stage (128),
 * tiles_m, tiles_n, grid, group_m, threads per workgroup, the number of K
 * parts and the stages per part.  The small-output kernel (a grid of
 * tiles_m * tiles_n workgroups of 512 threads, group_m 1, no split) takes
 * 16 x 16 tiles where M <= 16, else 32 x 32 where those number at least
 * num_cus, else 32 x 16 where those do, else 16 x 16; the tiled kernel
 * 256 x 256 tiles.  The split rule is dense_gemm_plan's for 256-wide
 * tiles with the FP8 kernel's costs: the estimate ceil(stages / p) * 100 +
 * 1000 + 5 * f * p * r against stages * 100 unsplit.
 * DENSE_GEMM_BAD_ARG on a bad argument, DENSE_GEMM_TOO_LARGE when the
 * tiles overflow 32-bit task numbers. */
dense_gemm_status gemm_nt_e4m3_mx_plan(int64_t M, int64_t N, int64_t K, int64_t num_cus,
                                       int64_t* out);

/* The workgroup-to-task permutation of the persistent grid: workgroup b
 * (dispatched to XCD b mod num_xcds) takes slot dense_gemm_xcd_slot(...) of
 * the task order, so that workgroups that share an XCD's L2 take adjacent
 * tasks.  A bijection of [0, grid).  Returns -1 on a bad argument. */
int64_t dense_gemm_xcd_slot(int64_t b, int64_t grid, int64_t num_xcds);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_H */
