/*
 * skinny_gemm.h -- C ABI of the MI355X (gfx950) BF16 skinny GEMM library
 * (libskinny_gemm_bf16.so).
 *
 * The operation, F.linear on bfloat16 at decode token counts:
 *
 *     y[m, n] = bf16_rne( sum_k x[m, k] * W[n, k] ),   m < M, n < N, k < K,
 *
 * with float32 accumulation and one round-to-nearest-even step to bfloat16 at
 * the end. It is the skinny GEMM of vLLM PR #62949 (SM121 skinny GEMM plans;
 * Overview and Claims: BF16 attention, shared-expert and LM-head projections at
 * M = 1/2/4, checked against F.linear in section Validation) and vLLM PR #65306
 * (SM90 skinny GEMM plans; Overview: 1..4 tokens; Details: one launch per GEMM,
 * no separate reduce kernel). The paired entry point is the batched f_b_proj /
 * g_b_proj projection of vLLM PR #57617 (paired KDA gate projections; section
 * "Purpose and source": two same-shape BF16 projections in one batched call).
 *
 * Conventions shared by every entry point below:
 *  - Pointers x, W, y are DEVICE pointers to bfloat16 values stored as raw
 *    16-bit patterns. Layouts are row-major and contiguous: x is [M][K], W is
 *    [N][K] (the nn.Linear weight layout, one output feature per row), y is
 *    [M][N]. No bias, no scaling.
 *  - The caller owns every buffer. The library never allocates, frees or
 *    synchronises in a compute call; it enqueues exactly one kernel on
 *    `stream` (0 = the null stream) and returns (the first allocation-free
 *    split-K call on a GPU enqueues one more, see below). Calls are therefore
 *    legal inside HIP graph capture. y must not overlap x or W (or, for the
 *    pair, each other). The only device memory the library owns is the static
 *    split-K workspace of skinny_gemm_bf16_split_k_noalloc, one per GPU.
 *  - Sizes: 0 <= M <= 8; N >= 0; K >= 0. M == 0 or N == 0 is a no-op that
 *    returns SKINNY_OK (pointers may then be NULL). K == 0 writes +0 to all of
 *    y (the empty sum). M = 1..4 is the decode range the cited plans cover;
 *    M = 5..8 runs the same kernel families (not the MFMA one, whose A operand
 *    has 4 rows) with tuned plans for the decode shapes. M > 8 is rejected with
 *    SKINNY_ERR_INVALID_ARG; the caller keeps its general GEMM.
 *  - Fast path: x and W 16-byte aligned, K % 8 == 0 (128-bit weight loads)
 *    and the output span ((M - 1) * ldy + N) * (output element bytes) < 2^31,
 *    where ldy = N except for the strided pair. Anything else runs a correct
 *    element-wise path; it is not an error (an explicit plan that cannot run
 *    returns SKINNY_ERR_INVALID_ARG or SKINNY_ERR_UNSUPPORTED instead).
 *  - Errors are returned, never raised or aborted: arguments are validated
 *    before anything is enqueued, and nothing is written on error. Only
 *    gfx950 devices are supported (others: SKINNY_ERR_UNSUPPORTED).
 *  - Results are deterministic: the same inputs and plan give the same bits on
 *    every call, eagerly or replayed from a graph. The reduction order depends
 *    only on the plan's (lanes_per_row, chunks, k_split) and K, so plans that
 *    share those give identical bits, and the pair gives the same bits as two
 *    single calls with the same plan.
 *  - Thread safety: every entry point may be called from any host thread; the
 *    only shared host state is caches filled on first use under a lock or
 *    with atomics (device properties; per kernel, its occupancy, static LDS
 *    size and raised LDS limit; per (device, N, K, M, single or pair), the
 *    resolved launch of the default plan, written once and then read without
 *    a lock, so that a repeated call does no table lookup; per device, the
 *    address of the static split-K workspace). Device-side, split-K calls that
 *    share a workspace (a caller's, or the static one) must not overlap.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
typedef enum skinny_status {
    SKINNY_OK = 0,
    SKINNY_ERR_INVALID_ARG = -1,     /* null pointer, size out of range, overlap, bad plan */
    SKINNY_ERR_UNSUPPORTED = -2,     /* no usable device, device is not gfx950, or no compiled
                                        variant matches the requested plan */
    SKINNY_ERR_NOT_INITIALIZED = -3, /* reserved: no entry point currently needs prior init */
    SKINNY_ERR_LAUNCH = -4           /* the HIP runtime refused the launch */
} skinny_status_t;

/* Kernel families a plan can name. */
typedef enum skinny_kind {
    SKINNY_KIND_FIXED_K = 1, /* K fixed at compile time = k_split*lanes_per_row*8*chunks;
                                x in registers or LDS, tiles optionally software-pipelined */
    SKINNY_KIND_LOOP_K = 2,  /* any K % 8 == 0; x staged in LDS; chunks = loads in flight per row */
    SKINNY_KIND_SCALAR = 3,  /* any K, any alignment; element-wise loads */
    SKINNY_KIND_MFMA = 4,    /* K % (128*k_split*chunks) == 0; 4-row groups on the matrix
                                cores (v_mfma_f32_4x4x4_16b_bf16), x staged in LDS,
                                chunks = loads per group per K batch, lanes_per_row = 16 */
    SKINNY_KIND_SPLIT_K = 5  /* cross-block split-K, only through skinny_gemm_bf16_split_k*:
                                K = k_split*lanes_per_row*8*chunks, k_split blocks per row
                                tile each take one K slice, partials in a workspace */
} skinny_kind_t;

/* One launch configuration ("plan"): the knobs of the plan tuple of vLLM PR
 * #62949 (SM121 skinny GEMM plans), section Details -- block size, outputs per
 * block, K unroll, vector width, static K -- recast for 64-wide wavefronts.
 * Vector width is fixed at 8 bfloat16 (one 128-bit load per lane). */
typedef struct skinny_plan {
    int32_t kind;              /* skinny_kind_t */
    int32_t threads_per_block; /* 64 * waves per block */
    int32_t lanes_per_row;     /* lanes sharing one W row in a load instruction: 8, 16, 32, 64 */
    int32_t chunks;            /* FIXED_K: 16-byte loads per lane per row; LOOP_K: loads per
                                  lane per row kept in flight (K unroll) */
    int32_t rows_per_wave;     /* row groups a wave processes per tile (outputs per wave =
                                  rows_per_wave * 64 / lanes_per_row) */
    int32_t k_split;           /* waves of one block that split a row's K range (1, 2, 4, 8);
                                  partial sums meet in LDS, summed in fixed order */
    int32_t nontemporal;       /* 1: W is read with the non-temporal cache hint */
    int32_t grid_blocks;       /* 0: a persistent grid that fills the device once (compute
                                  units x blocks resident per unit), each block looping over
                                  tiles; > 0: at most this many blocks (a value >= the tile
                                  count gives one block per tile) */
    int32_t x_in_lds;          /* FIXED_K: 1 = x staged once per block in LDS, each chunk's
                                  pieces read back when the chunk is multiplied; 2 = the
                                  same, read one chunk ahead (one row per wave, M >= 2);
                                  0 = each lane keeps its slice of x in registers;
                                  LOOP_K, MFMA: always 1; SCALAR: always 0 */
    int32_t prefetch;          /* FIXED_K, MFMA: 1 = the next tile's (MFMA: the next K batch's)
                                  weights are loaded while the current one is consumed (two
                                  register sets); 0 = one at a time. FIXED_K also 2 = rolling:
                                  one register set, each 16-byte chunk of the next tile is
                                  loaded as soon as the same chunk of the current tile has been
                                  multiplied. Other kinds: always 0 */
} skinny_plan_t;

/* Checks that `device` is a gfx950 GPU, caches its properties and looks up that
 * device's copy of the static workspace of skinny_gemm_bf16_split_k_noalloc (with
 * the device made current for the lookup, the caller's device restored after).
 * Enqueues no work and allocates nothing. Optional: every compute call performs
 * the same steps lazily on the current device. Idempotent. Returns SKINNY_OK,
 * SKINNY_ERR_INVALID_ARG (no such device), SKINNY_ERR_UNSUPPORTED (not gfx950)
 * or SKINNY_ERR_LAUNCH (the runtime refused the workspace lookup). */
int skinny_gemm_init(int device);

/* y = x . W^T with the plan the library's table holds for (N, K, M) on this
 * architecture, or its default plan when the table has no entry. The table is
 * keyed like the plan tables of vLLM PR #65306 (SM90 skinny GEMM plans),
 * section Details: architecture + local (N, K) + M. */
int skinny_gemm_bf16(const void *x, const void *W, void *y,
                     int M, int N, int K, hipStream_t stream);

/* The paired projection: y0 = x . W0^T and y1 = x . W1^T, both [N][K] weights
 * applied to the one shared x, in ONE kernel launch (vLLM PR #57617, paired KDA
 * gate projections, section "Purpose and source"; LMDeploy PR #4968, GLM-5.3
 * Flash support, the batched f_b/g_b row of its operator-level gains table).
 * Same conventions as skinny_gemm_bf16; y0 and y1 must not overlap each other,
 * x, W0 or W1. */
int skinny_gemm_bf16_pair(const void *x, const void *W0, const void *W1,
                          void *y0, void *y1, int M, int N, int K, hipStream_t stream);

/* The paired projection in the form the f_b_proj / g_b_proj pair actually takes:
 * each weight has its own input, two row-strided views of one merged activation
 * (vLLM PR #57617, paired KDA gate projections, section "Controlled follow-up": a
 * narrow -> unflatten -> transpose view over the merged f_a/g_a output feeding one
 * batched matmul; LMDeploy PR #4968, section Optimizations: f_a/g_a merged, f_b/g_b
 * batched). y0 = x0 . W0^T and y1 = x1 . W1^T in ONE launch, where row m of x0 is
 * the K elements at x0 + m*ldx, likewise x1, and row m of y0 / y1 is the N
 * elements at y0 + m*ldy / y1 + m*ldy. Typical use: a merged [M][2K] activation
 * with x0 = base, x1 = base + K, ldx = 2K, and a merged [M][2N] output with
 * y1 = y0 + N, ldy = 2N. ldx >= K and ldy >= N (else SKINNY_ERR_INVALID_ARG);
 * x0/x1 may overlap each other (they are only read); y0 and y1 must share no
 * element with each other, x0, x1, W0 or W1. The fast path needs x0, x1, W0, W1
 * 16-byte aligned and ldx % 8 == 0. Other conventions as skinny_gemm_bf16_pair. */
int skinny_gemm_bf16_pair_strided(const void *x0, const void *x1, int ldx,
                                  const void *W0, const void *W1,
                                  void *y0, void *y1, int ldy,
                                  int M, int N, int K, hipStream_t stream);
int skinny_gemm_bf16_pair_strided_ex(const void *x0, const void *x1, int ldx,
                                     const void *W0, const void *W1,
                                     void *y0, void *y1, int ldy,
                                     int M, int N, int K, const skinny_plan_t *plan,
                                     hipStream_t stream);

/* As skinny_gemm_bf16 / _pair, with an explicit plan (used by the plan sweep
 * and by tests). The plan must name a compiled variant (see
 * skinny_gemm_num_variants) compatible with K: for FIXED_K, K must equal
 * k_split*lanes_per_row*8*chunks. A FIXED_K or LOOP_K plan given misaligned
 * pointers or K % 8 != 0 returns SKINNY_ERR_INVALID_ARG. grid_blocks may be
 * any value >= 0 for any variant. */
int skinny_gemm_bf16_ex(const void *x, const void *W, void *y,
                        int M, int N, int K, const skinny_plan_t *plan, hipStream_t stream);
int skinny_gemm_bf16_pair_ex(const void *x, const void *W0, const void *W1,
                             void *y0, void *y1, int M, int N, int K,
                             const skinny_plan_t *plan, hipStream_t stream);

/* y = x . W^T with float32 outputs: the float32 accumulation is stored without the
 * bfloat16 rounding. This is the epilogue of the router gate (288, 4096), the one
 * BF16-input projection with an fp32 output that vLLM PR #62949 (SM121 skinny GEMM
 * plans), section Validation, leaves on cuBLAS. x and W as in skinny_gemm_bf16; y
 * is a DEVICE pointer to M*N float32 values, row-major [M][N], 4-byte aligned, not
 * overlapping x or W. Same plans, sizes, errors and stream semantics as
 * skinny_gemm_bf16 / skinny_gemm_bf16_ex (K == 0 writes +0.0f). */
int skinny_gemm_bf16_f32out(const void *x, const void *W, float *y,
                            int M, int N, int K, hipStream_t stream);
int skinny_gemm_bf16_f32out_ex(const void *x, const void *W, float *y,
                               int M, int N, int K, const skinny_plan_t *plan, hipStream_t stream);

/* The plan skinny_gemm_bf16 would use for (N, K, M) with 16-byte aligned
 * pointers. Writes *out; returns 1 if it comes from the tuned table, 0 if it is
 * the default plan, or SKINNY_ERR_INVALID_ARG. Host-only: needs no device. */
int skinny_gemm_get_plan(int N, int K, int M, skinny_plan_t *out);

/* Enumerates the compiled variants (grid_blocks = 0 in each). A variant covers
 * M = 1..8 except an M whose instance would exceed its register budget (MFMA
 * variants cover M = 1..4 only); a plan naming it at such an M returns
 * SKINNY_ERR_UNSUPPORTED. skinny_gemm_get_variant returns SKINNY_OK or
 * SKINNY_ERR_INVALID_ARG for an index out of range. Host-only. */
int skinny_gemm_num_variants(void);
int skinny_gemm_get_variant(int index, skinny_plan_t *out);

/* ---- Cross-block split-K ------------------------------------------------------
 * y = x . W^T in ONE launch where the K range of every row is cut into S slices
 * (plan.k_split) that S different blocks take: the single-launch form of the
 * split-K + reduce kernel pair that vLLM PR #65306 (SM90 skinny GEMM plans),
 * section Details, counts against cuBLAS on its small-N / large-K shapes. Each
 * block stores its float32 partial sums in a workspace with device-coherent
 * stores, waits for them and bumps a per-tile arrival counter; the last block of
 * a row tile to arrive reads the S partials with device-coherent loads, adds them
 * in slice order 0..S-1 and writes bfloat16 y. No block waits for another. The result equals, bit for bit, that of the FIXED_K plan with the
 * same (lanes_per_row, chunks) and k_split = S.
 *
 * Plans: kind SKINNY_KIND_SPLIT_K, a variant from skinny_gemm_split_k_get_variant
 * with k_split = S >= 1 set by the caller, threads_per_block a multiple of 64 in
 * 64..512, nontemporal 1, grid_blocks 0 (one block per row tile and slice),
 * x_in_lds 0, prefetch 0; K must equal S * lanes_per_row * 8 * chunks. plan ==
 * NULL picks a default (256 threads, one row per wave, S in 4, 2, 8 order) or
 * returns SKINNY_ERR_UNSUPPORTED when no compiled slice fits K.
 *
 * Same conventions as skinny_gemm_bf16 for x, W, y, M, N, K and stream, except:
 * x and W must be 16-byte aligned and K % 8 == 0 (there is no element-wise
 * path: SKINNY_ERR_INVALID_ARG otherwise), K > 0, and only bfloat16 output. */

/* Bytes of workspace a split-K call needs: 64 KiB of 32-bit arrival counters
 * (16384, one per row tile; calls with more tiles are refused), then S*M*N
 * float32 partials. plan == NULL: the default plan. Returns 0 for arguments no
 * call accepts. */
size_t skinny_gemm_split_k_workspace_bytes(int M, int N, int K, const skinny_plan_t *plan);

/* Split-K with a caller-owned workspace: a DEVICE pointer, 256-byte aligned, of
 * at least skinny_gemm_split_k_workspace_bytes() bytes, overlapping none of x, W,
 * y. Its first 64 KiB (the counters) must be zero before the first call: fill the
 * workspace with zeros once, when it is allocated. Every complete call leaves the
 * counters zero again and writes partials only after them, which need no
 * clearing, so one workspace serves any later call it is large enough for,
 * eagerly or from a graph replay. Calls that may run at the same time (other
 * streams) must not share a workspace. Refused (SKINNY_ERR_INVALID_ARG): a
 * missing, misaligned, too small or overlapping workspace; more than 16384 row
 * tiles. */
int skinny_gemm_bf16_split_k(const void *x, const void *W, void *y, int M, int N, int K,
                             const skinny_plan_t *plan, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Split-K for callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * computation and result as skinny_gemm_bf16_split_k, on the library's own static
 * workspace instead of a caller's. That workspace is one device array per GPU, in
 * the same layout (64 KiB of counters, then 4 MiB of partials), held from the
 * library's load until the process ends; a call whose S*M*N exceeds 2^20, or that
 * has more than 16384 row tiles, returns SKINNY_ERR_INVALID_ARG. skinny_gemm_init
 * looks up each GPU's copy (else the first call on that GPU does); the first call
 * on a GPU also enqueues one small kernel on `stream` that zeroes the copy's
 * counters. No call allocates or frees memory. Every call on a GPU
 * shares that GPU's copy, so calls that may overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller. */
int skinny_gemm_bf16_split_k_noalloc(const void *x, const void *W, void *y, int M, int N, int K,
                                     const skinny_plan_t *plan, hipStream_t stream);

/* The compiled split-K variants (k_split = 0 in each: S is chosen per call), and
 * the default plan for a shape. Host-only. */
int skinny_gemm_split_k_num_variants(void);
int skinny_gemm_split_k_get_variant(int index, skinny_plan_t *out);
int skinny_gemm_split_k_default_plan(int M, int N, int K, skinny_plan_t *out);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *skinny_gemm_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int skinny_gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */
