/*
 * bst.h -- C ABI of the swizzled tiled GEMM library for AMD MI355X (gfx950).
 *
 * C = A . B with a GemmIdentityBlockSwizzle-style block -> tile scheduler
 * ("Block Scheduler Code Explained", CATLASS docs: s4.1 loop counts, s4.4
 * batch index, s4.5 Zn / Nz windows of width SwizzleOffset with snake
 * reversal, s4.6 tail-tile shapes, s6 runtime offset and direction), in four
 * forms: plain, batched, grouped slice-M, and int8 with per-token /
 * per-channel dequant (the workloads that "Block Dispatch Policies", CATLASS
 * docs, lists as examples of its dispatch policies).
 *
 * Conventions for every entry point
 *  - All matrices are row-major: A[M][lda] with lda >= K, B[K][ldb] with
 *    ldb >= N, C[M][ldc] with ldc >= N (leading dimensions in elements).
 *    Base pointers must be 16-byte aligned and every leading dimension and
 *    batch stride must be a whole number of 16-byte units (BST_E_ALIGN).
 *  - Pointers named *_dev are device pointers; the caller owns every buffer
 *    and the stream.  The library never allocates, frees or synchronises in
 *    a call: work is enqueued on `stream` (a hipStream_t, NULL = the null
 *    stream) and the call returns at once.
 *  - Validation happens on the host before any launch; on a non-OK status
 *    nothing was enqueued and bst_last_error() describes the problem.
 *  - M == 0, N == 0 or batch == 0 (no output) is a successful no-op.
 *    K == 0 writes zeros (dequant of zero is zero).
 *  - Results do not depend on the schedule (tile order, split, remap, grid);
 *    the tile shape and the split only change the fp32 summation order.
 *  - Calls that share a workspace must be ordered (same stream or synced).
 */
#ifndef BST_H
#define BST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bst_status {
  BST_OK = 0,
  BST_E_INVAL = -1,        /* bad argument: null pointer, negative or too-large size,
                              leading dimension < row length, offset 0, bad direction,
                              MX with K % 32 != 0, int8 with K > 131071 */
  BST_E_UNSUPPORTED = -2,  /* no compiled kernel for this dtype pair / tile */
  BST_E_ALIGN = -3,        /* base pointer or stride not 16-byte aligned */
  BST_E_WORKSPACE = -4,    /* workspace missing or smaller than bst_workspace_bytes() */
  BST_E_HIP = -5           /* the HIP runtime reported an error (message captured) */
} bst_status;

typedef enum bst_dtype {
  BST_F16 = 1,     /* IEEE binary16 */
  BST_BF16 = 2,    /* bfloat16 */
  BST_E4M3 = 3,    /* OCP FP8 E4M3 "fn" (no inf, max 448), unscaled */
  BST_MXE4M3 = 4,  /* OCP FP8 E4M3 with one E8M0 scale per 32 consecutive K values */
  BST_I8 = 5,      /* int8 */
  BST_I32 = 6,     /* int32 (raw int8 accumulators) */
  BST_F32 = 7,     /* binary32 */
  /* not dtypes: they make every int32 value a valid bst_dtype, so that the
     library can read and reject any value a caller passes */
  BST_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  BST_DTYPE_RANGE_MAX_ = 2147483647
} bst_dtype;

typedef enum bst_direction {
  BST_ZN = 0,      /* windows of swizzle_offset tile-rows, M index fastest inside (s4.5) */
  BST_NZ = 1,      /* windows of swizzle_offset tile-columns, N index fastest inside */
  BST_RASTER = 2   /* row-major over tiles, no windows, no snake (comparison baseline) */
} bst_direction;

/* Schedule of one call.  Only tile_m / tile_n and the swizzle fields decide
 * the task -> tile map; the others are performance knobs. */
typedef struct bst_sched {
  uint32_t tile_m, tile_n;     /* output tile (the scheduler's tileMN); 0 = default */
  uint32_t tile_k;             /* K depth of one pipeline stage; 0 = the dtype's only value
                                  (64 for 16-bit, 128 for 8-bit operands) */
  uint32_t swizzle_offset;     /* window width in tiles, >= 1 (SwizzleOffset, s2.1) */
  uint32_t swizzle_direction;  /* bst_direction (SwizzleDirection, s2.1; RASTER added) */
  uint32_t split_k;            /* K slices per tile: 1 = off, 0 = automatic */
  uint32_t xcd_remap;          /* 0: workgroup w takes tasks w, w+G, ...; 1: workgroups are
                                  renumbered so that each XCD (accelerator die, own L2)
                                  takes a contiguous range of task indices */
  uint32_t grid;               /* persistent workgroups; 0 = fill every CU */
  uint32_t path;               /* kernel family: 1 = register-staged (any shape);
                                  2 = LDS-DMA pipeline, one workgroup per CU with a deep
                                  pipeline (K and N whole 16-byte chunks, MX K a multiple of
                                  128, and a tile's rows of A, B and C each within 2 GiB;
                                  BST_E_UNSUPPORTED otherwise); 3 = LDS-DMA pipeline with
                                  two resident workgroups per CU and two stages, so that one
                                  workgroup's epilogue and set-up overlap the other's K loop
                                  (fp16 / bf16 / int8 at 128x128, plain, batched and grouped
                                  slice-M; MX-fp8 at 128x128, plain; BST_E_UNSUPPORTED
                                  otherwise); 0 = automatic: path 1
                                  when the layout rules out the LDS-DMA family, else path 3
                                  where it exists and the launch has more work units than CUs,
                                  else path 2.  Paths 2 and 3 add the same products in the
                                  same order: their results are bit-identical (up to the sign
                                  of an exactly zero floating-point sum). */
  uint32_t shuffle_k;          /* 1: ShuffleK (a policy flag of the Preload dispatch policies,
                                  "Block Dispatch Policies"): the K loop of task t starts at
                                  stage t mod S of its S stages and wraps around, so that tiles
                                  running together read different K slices.  Applied by the
                                  LDS-DMA family to tasks of whole stages whose count is the
                                  launch's full slice (not to a shorter last slice, nor to
                                  slice-K groups); others run in order.  0 = off.  Results
                                  differ from 0 only by fp32 summation order (int8:
                                  bit-identical). */
  uint32_t dynamic;            /* 1: dynamic task allocation ("Block Scheduler Code Explained",
                                  s1): after a first round of one unit per workgroup, the
                                  units go to eight queues, one per XCD; each workgroup takes
                                  tickets from its own XCD's queue, then from the others, so
                                  uneven tiles and groups even out.  Needs the workspace's
                                  counter area (bst_workspace_bytes is never 0 with it).
                                  LDS-DMA family only; results are identical to 0.
                                  0 = static stride. */
  uint32_t preload;            /* 1: block preloading (a policy of the Preload dispatch
                                  policies, "Block Dispatch Policies"): a workgroup issues the
                                  first stage of its next task before the current task's
                                  epilogue, which stages through a buffer it does not use.
                                  LDS-DMA family with the static stride only (with dynamic
                                  allocation the next task is known only after the
                                  epilogue); results are identical to 0. */
} bst_sched;

/*
 * bst_gemm -- C = A . B for one problem (the basic matmul that "Block
 * Dispatch Policies" lists under its ping-pong policy), its output tiles
 * visited in the order of the swizzled block scheduler ("Block Scheduler
 * Code Explained", s4.3 GetCoreLoops for the task count, s4.5
 * GetBlockCoord for each task's tile, s4.6 GetActualBlockShape for the tail
 * tiles of the last tile-row and tile-column).
 *   ab: BST_F16 / BST_BF16 (c: BST_F16, BST_BF16 or BST_F32), BST_E4M3 /
 *   BST_MXE4M3 (c: BST_BF16, BST_F16 or BST_F32), BST_I8 (c: BST_I32 raw
 *   accumulators, or BST_F32 / BST_BF16 / BST_F16 of the accumulator).
 *   scale_a_dev, scale_b_dev: BST_MXE4M3 only, else NULL.  scale_a is
 *   uint8 E8M0 [M][K/32] (row-major, one scale per row and 32-wide K block),
 *   scale_b is uint8 E8M0 [K/32][N].  K must be a multiple of 32.
 *   Element (i, j) = sum over K blocks of 2^(sa-127) * 2^(sb-127) * (sum of
 *   the block's products).
 *   Accumulation is fp32 (int32 for int8); outputs are rounded to nearest
 *   even.  ws / ws_bytes: workspace of at least bst_workspace_bytes(...)
 *   bytes when the (possibly automatic) split_k is above 1 or dynamic
 *   allocation is on, else may be NULL / 0.  Layout: a counter area of
 *   73728 bytes (one uint32 per tile, at most 16384 tiles take a split;
 *   then 8 KiB of work-queue counters) followed by the partial tiles.
 *   The counter area must be zero before the first use of a workspace;
 *   every call that runs to completion leaves it zero again, so one
 *   workspace serves calls of any shape in stream order.
 */
bst_status bst_gemm(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K,
                    const void* A_dev, int64_t lda, const void* B_dev, int64_t ldb,
                    void* C_dev, int64_t ldc, const uint8_t* scale_a_dev,
                    const uint8_t* scale_b_dev, const bst_sched* sched, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * bst_gemm_noalloc -- bst_gemm for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operands, schedule and results, and no workspace
 * argument.  The split-K partials and counters and the dynamic-allocation
 * queues live in a static scratch array inside the library: 32 MiB of
 * device memory per GPU, held from the library's load until the process
 * ends, addressed once per device (hipGetSymbolAddress) on the first call
 * there, which also clears its counter area on `stream`.  The call itself
 * allocates and frees nothing.  A schedule needing more than 32 MiB
 * (bst_workspace_bytes) returns BST_E_WORKSPACE before anything is
 * enqueued.  Every call on one GPU shares that GPU's scratch and leaves its
 * counters zero again when it completes: calls that overlap on one GPU
 * (different streams, or host threads without ordering) race and must not
 * be issued.
 */
bst_status bst_gemm_noalloc(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K,
                            const void* A_dev, int64_t lda, const void* B_dev, int64_t ldb,
                            void* C_dev, int64_t ldc, const uint8_t* scale_a_dev,
                            const uint8_t* scale_b_dev, const bst_sched* sched, void* stream);

/*
 * bst_gemm_add -- C = A . B + X (the matmul-add example that "Block Dispatch
 * Policies" lists under its ping-pong policy; reading: X has C's shape and
 * dtype c).  Same operands, scales, schedule and workspace as bst_gemm.
 *   X_dev: [M][ldx] of dtype c, 16-byte aligned, ldx >= N with ldx * sizeof
 *   a 16-byte multiple; it may be C itself (C += A . B).  Each output adds
 *   X in fp32 (int32 for BST_I32, wrapping) to the fp32 accumulator and is
 *   rounded once.  Errors as bst_gemm, plus BST_E_INVAL for a NULL X or a
 *   small ldx, BST_E_ALIGN for a misaligned X, and BST_E_UNSUPPORTED for a
 *   tile without a matmul-add kernel (fp16 / bf16: 64x64, 128x128; MX-fp8:
 *   64x128, 128x128; fp8 and int8: 128x128) or for operands the LDS-DMA
 *   kernels cannot take (K or N not in whole 16-byte chunks, path 1).
 */
bst_status bst_gemm_add(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K,
                        const void* A_dev, int64_t lda, const void* B_dev, int64_t ldb,
                        const void* X_dev, int64_t ldx, void* C_dev, int64_t ldc,
                        const uint8_t* scale_a_dev, const uint8_t* scale_b_dev,
                        const bst_sched* sched, void* ws, size_t ws_bytes, void* stream);

/*
 * bst_gemm_padded -- bst_gemm for operands whose rows are not whole 16-byte
 * chunks or whose base is not 16-byte aligned (the padding matmul example
 * that "Block Dispatch Policies" lists under its ping-pong policy; reading:
 * repack the operands into an aligned, zero-padded layout, then run the
 * GEMM).  A [M][lda] and B [K][ldb] may have any leading dimension >= K / N
 * and any element-aligned base; the call copies them into the workspace
 * with rows rounded up to whole 16-byte chunks (zeros in the padding), B
 * with K rounded up the same way (zero rows), and runs bst_gemm on the
 * copies at that K, in stream order: the added products are exact zeros,
 * and the copies fit the LDS-DMA kernels whenever N is a whole number of
 * 16-byte chunks.  C, the MX scales and the rest are as for bst_gemm (C
 * stays 16-byte aligned).  ws: at least bst_workspace_bytes(2, ab, 1, M,
 * N, K, sched) bytes, 16-byte aligned (BST_E_WORKSPACE / BST_E_ALIGN
 * otherwise); the call owns it until the GEMM has run.  Every argument is
 * checked before the copies are enqueued.
 */
bst_status bst_gemm_padded(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K,
                           const void* A_dev, int64_t lda, const void* B_dev, int64_t ldb,
                           void* C_dev, int64_t ldc, const uint8_t* scale_a_dev,
                           const uint8_t* scale_b_dev, const bst_sched* sched, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * bst_batched_gemm -- C_b = A_b . B_b for b in [0, batch), with
 * A_b = A + b*strideA, B_b = B + b*strideB, C_b = C + b*strideC (strides in
 * elements).  The task index spans batch x tiles; the batch index of task t
 * is t / (tiles per problem) (s4.4 GetBatchIdx).  Same dtypes as bst_gemm
 * except BST_MXE4M3.  With batch > 1 the batches of C may not overlap:
 * strideC >= (M-1)*ldc + N (BST_E_INVAL otherwise); A and B batches may.
 */
bst_status bst_batched_gemm(bst_dtype ab, bst_dtype c, int64_t batch, int64_t M, int64_t N,
                            int64_t K, const void* A_dev, int64_t lda, int64_t strideA,
                            const void* B_dev, int64_t ldb, int64_t strideB, void* C_dev,
                            int64_t ldc, int64_t strideC, const bst_sched* sched, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * bst_grouped_gemm_slice_m -- G independent problems stacked along M that
 * share N and K: group g owns rows [P_g, P_g + group_m[g]) of A and C, where
 * P_g = sum of group_m[h] for h < g, and uses B_g = B + g*strideB
 * ([K][ldb]).  group_m_dev is a device int32[G] and is never read by the
 * host; entries < 0 count as 0, and a group is cut to the rows still left
 * of total_m (the rows allocated in A and C), so nothing at or beyond row
 * total_m is read or written.  Tasks are the
 * groups' tile ranges concatenated in group order; inside a group the
 * scheduler is re-targeted to (group_m[g], N) (s4.2 Update).
 *   ab = BST_I8: c = BST_I32 (raw), or BST_BF16 / BST_F16 / BST_F32 with
 *   optional dequant: when row_scale_dev (f32 [total_m], per token) and
 *   col_scale_dev (f32 [G][N], per group and channel) are both given,
 *   out = round(float(acc) * row_scale[r] * col_scale[g][j]) with each
 *   product rounded to fp32.  ab = BST_F16 / BST_BF16: no scales.
 *   1 <= G <= 1024.
 */
bst_status bst_grouped_gemm_slice_m(bst_dtype ab, bst_dtype c, int32_t G,
                                    const int32_t* group_m_dev, int64_t total_m, int64_t N,
                                    int64_t K, const void* A_dev, int64_t lda,
                                    const void* B_dev, int64_t ldb, int64_t strideB,
                                    void* C_dev, int64_t ldc, const float* row_scale_dev,
                                    const float* col_scale_dev, const bst_sched* sched,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * bst_grouped_gemm_slice_k -- G problems that cut one K dimension into
 * consecutive groups (the grouped-matmul-slice-K example, with and without
 * per-token dequant, that "Block Dispatch Policies" lists under its
 * PreloadAsync policies; reading: each group is its own product with its
 * own output).  Group g owns K indices [Q_g, Q_g + group_k[g]) with Q_g the
 * sum of the earlier groups' sizes: columns of A (row-major [M][lda],
 * lda >= total_k) and rows of B (row-major [total_k][ldb]).  Its output is
 * C_g = A[:, Q_g : Q_g + k_g] . B[Q_g : Q_g + k_g, :], an M x N matrix at
 * C + g*strideC ([M][ldc]); groups' outputs may not overlap (strideC >=
 * (M-1)*ldc + N when G > 1, BST_E_INVAL otherwise).  Every group shares M
 * and N, so the tasks are numbered like the batches of a batched problem
 * (group of task t = t / tiles per group, s4.4 GetBatchIdx) and
 * bst_tile_map with batch = G dumps their map.
 *   group_k_dev: device int32[G] (never read by the host); entries < 0
 *   count as 0 and a group is cut to the K still left of total_k, so
 *   nothing past column / row total_k is read.  An empty group's output
 *   is zeros.  The LDS-DMA kernels (path 2, the automatic choice when the
 *   layout allows) need every group to start and end on a whole 16-byte
 *   chunk of A's rows (sizes multiples of 8 for 16-bit operands, 16 for
 *   int8); a group that does not is not computed and its whole output
 *   reads NaN (INT32_MIN for raw int32 accumulators), as does every later
 *   group whose start it shifts.  The register-staged kernels (path 1)
 *   take groups of any size.
 *   ab = BST_I8: c = BST_I32 (raw), or BST_BF16 / BST_F16 / BST_F32 with
 *   optional dequant: with row_scale_dev (f32 [G][M], per group and token
 *   row) and col_scale_dev (f32 [G][N], per group and channel) both given,
 *   out = round(float(acc) * row_scale[g][i] * col_scale[g][j]) with each
 *   product rounded to fp32.  ab = BST_F16 / BST_BF16: no scales.
 *   1 <= G <= 1024.  The split-K option (sched->split_k) cuts every group's
 *   K range into that many slices of whole stages on the device (0 = judged
 *   from the mean group size); ws as for bst_gemm, sized by
 *   bst_workspace_bytes(3, ab, G, M, N, total_k, sched).
 */
bst_status bst_grouped_gemm_slice_k(bst_dtype ab, bst_dtype c, int32_t G,
                                    const int32_t* group_k_dev, int64_t total_k, int64_t M,
                                    int64_t N, const void* A_dev, int64_t lda,
                                    const void* B_dev, int64_t ldb, void* C_dev, int64_t ldc,
                                    int64_t strideC, const float* row_scale_dev,
                                    const float* col_scale_dev, const bst_sched* sched,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * bst_quant_gemm_per_token -- the quantised matmul with per-token dequant
 * ("Block Dispatch Policies" lists quant-matmul and per-token-dequant
 * examples under its PreloadAsync policies; reading: one problem, the
 * scales applied to the int32 accumulators in the epilogue):
 * int8 A[M][K] . int8 B[K][N] with int32
 * accumulation and, for c = BST_BF16 / BST_F16 / BST_F32, the dequant
 * out = round(float(acc) * row_scale[i] * col_scale[j]) (row_scale f32 [M]
 * per token, col_scale f32 [N] per channel, both device pointers, both
 * required); c = BST_I32 writes the raw accumulators (scales ignored).
 */
bst_status bst_quant_gemm_per_token(int64_t M, int64_t N, int64_t K, const int8_t* A_dev,
                                    int64_t lda, const int8_t* B_dev, int64_t ldb,
                                    const float* row_scale_dev, const float* col_scale_dev,
                                    void* C_dev, int64_t ldc, bst_dtype c,
                                    const bst_sched* sched, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * bst_tile_map -- the task -> tile map as the GPU computes it, with the
 * device scheduler the GEMM kernels use ("Block Scheduler Code Explained":
 * s4.4 GetBatchIdx, s4.5 GetBlockCoord, s4.6 GetActualBlockShape, with the
 * runtime offset and direction of s6).  For every task t of a batched
 * problem (batch x ceil(M/tile_m) x ceil(N/tile_n) tasks) writes 8 uint32
 * to out_dev[8t..8t+7]: {batch index, m, n, mActual, nActual, 0, XCC id of
 * the workgroup that ran it, that workgroup's index}.  `ab` selects the tile
 * defaults.  max_tasks bounds out_dev (BST_E_INVAL if too small).
 */
bst_status bst_tile_map(bst_dtype ab, int64_t batch, int64_t M, int64_t N,
                        const bst_sched* sched, uint32_t* out_dev, int64_t max_tasks,
                        void* stream);

/*
 * bst_grouped_tile_map -- as bst_tile_map for a grouped slice-M problem:
 * {group, m, n, mActual, nActual, first stacked row of the tile, XCC id,
 * workgroup}.  group_m_dev as in bst_grouped_gemm_slice_m; the task count
 * is only known on the device, so max_tasks must be at least
 * (ceil(total_m/tile_m) + G) * ceil(N/tile_n); unused records are left
 * untouched.  *
 */
bst_status bst_grouped_tile_map(bst_dtype ab, int32_t G, const int32_t* group_m_dev,
                                int64_t total_m, int64_t N, const bst_sched* sched,
                                uint32_t* out_dev, int64_t max_tasks, void* stream);

/*
 * bst_workspace_bytes -- workspace bytes a call with these arguments needs
 * (0 when the effective split_k is 1).  kind: 0 plain / batched (count =
 * batch), 1 grouped slice-M (count = G, M = total_m), 2 bst_gemm_padded
 * (count 1; the repacked operands plus the split-K workspace, never 0 for a
 * non-empty problem), 3 grouped slice-K (count = G, K = total_k).  Returns
 * 0 and sets the last error for invalid arguments.
 */
size_t bst_workspace_bytes(int kind, bst_dtype ab, int64_t count, int64_t M, int64_t N,
                           int64_t K, const bst_sched* sched);

/* bst_effective_sched -- fills *out with the schedule a call with these
 * arguments would run (defaults and automatic split resolved).  kind as for
 * bst_workspace_bytes (2: the GEMM bst_gemm_padded runs on its copies). */
bst_status bst_effective_sched(int kind, bst_dtype ab, int64_t count, int64_t M, int64_t N,
                               int64_t K, const bst_sched* sched, bst_sched* out);

/* bst_task_count -- tasks of the block scheduler for these sizes (s4.3
 * GetCoreLoops times the batch count, s4.4): kind 0 plain / batched
 * (count = batch) and kind 3 grouped slice-K (count = G): exactly
 * count * ceil(M/tile_m) * ceil(N/tile_n); kind 1 grouped slice-M (count =
 * G, M = total_m): the bound (ceil(total_m/tile_m) + G) * ceil(N/tile_n),
 * since the group sizes live on the device.  This is the record count bst_tile_map /
 * bst_grouped_tile_map need.  Tiles are the effective ones (defaults
 * resolved). */
bst_status bst_task_count(int kind, bst_dtype ab, int64_t count, int64_t M, int64_t N,
                          const bst_sched* sched, int64_t* tasks);

/* bst_set_clock_record -- measurement hook for the shader clock a GEMM runs
 * at.  While set (n > 0), every GEMM launched on the LDS-DMA kernels makes
 * each of its first n workgroups record, at dev_buf[4w .. 4w+3] (uint64,
 * device memory of at least 32 n bytes), the 100 MHz reference counter at
 * the workgroup's start and end, its shader cycles in between, and 1; the
 * shader clock is cycles / ((end - start) / 100 MHz).  n = 0 turns it off
 * (the kernels then only test a null pointer).  Process-wide: set it from
 * one thread while no GEMM is being enqueued.  BST_E_INVAL for n < 0 or a
 * NULL buffer with n > 0. */
bst_status bst_set_clock_record(void* dev_buf, int64_t n);

/* Message for the last non-OK status returned on this thread. */
const char* bst_last_error(void);

/* Library version string. */
const char* bst_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BST_H */
