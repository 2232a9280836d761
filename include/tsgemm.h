/*
 * tsgemm.h -- C ABI of the persistent, tile-scheduled dense GEMM for MI355X
 * (gfx950 / CDNA4).  Library: libtsgemm.so.
 *
 *   C[M,N] = A[M,K] * B[K,N]
 *
 * A, B and C are row-major and contiguous and share one 16-bit dtype (fp16 or
 * bf16); products accumulate in fp32 and each C element is rounded once to the
 * dtype (round to nearest, ties to even).  This is the product computed by the
 * persistent example of page "[Feature] Introduce tile scheduler #2441" (diff of
 * examples/gemm_sm100/gemm_tcgen5mma_ws_persistent.py: A[M,K] and B[K,N]
 * copied slab by slab into shared memory, accumulated into an fp32 tile, cast
 * and stored; checked against torch `a @ b` in main()).
 *
 * A fixed grid of persistent workgroups runs one loop each, driven by a tile
 * scheduler that owns the wave clock w: worker `wid` visits
 * tile_id = P*w + wid while tile_id < num_tiles, decoding it into (m_idx, n_idx)
 * in groups of `group_size` column blocks (same page: the manual tile walk that
 * PersistentTileScheduler(..., swizzle_size=group_size) replaces; the page's
 * conversation tab lists init / valid / next_tile and coord(tile_id)).  When
 * n_blocks is not a multiple of group_size the last group is narrower.
 *
 * Conventions (the page "tilelang" blog, section 1.3, shows the host stubs this
 * follows: init / call(A, B, C, stream) returning 0 or -1 with the message in
 * get_last_error(), and the argument checks of the lowered host function):
 *   - every int-returning call returns TSGEMM_OK (0) or a negative TSGEMM_E*
 *     code and then sets a message readable with tsgemm_last_error();
 *   - pointer arguments named A, B, C are DEVICE pointers, the caller owns
 *     them; `out` arguments of the schedule calls are HOST pointers;
 *   - the library keeps no pointer after a call returns; a plan is immutable
 *     once configured (create + the set_* calls), so concurrent runs of one
 *     plan on different streams are safe.
 */
#ifndef TSGEMM_H
#define TSGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tsgemm_plan tsgemm_plan; /* opaque, owned by the library */

/* TSGEMM_MXFP8: block-scaled FP8 inputs with bf16 output (tsgemm_run_mx). */
enum { TSGEMM_FP16 = 1, TSGEMM_BF16 = 2, TSGEMM_MXFP8 = 3 };

enum {
    TSGEMM_OK = 0,
    TSGEMM_EINVAL = -1,       /* malformed argument                              */
    TSGEMM_EUNSUPPORTED = -2, /* well-formed but outside the compiled kernels    */
    TSGEMM_EHIP = -3,         /* a HIP runtime call failed (no device, launch)   */
    TSGEMM_ENOMEM = -4        /* allocation failed                               */
};

/* Plan summary; every field is derived at create/configure time. */
typedef struct tsgemm_info {
    int64_t M, N, K;
    int32_t dtype;
    int32_t block_M, block_N, block_K;
    int32_t group_size;
    int32_t num_stages;      /* as requested                                         */
    int32_t lds_slots;       /* K-slabs resident in LDS: min(num_stages, LDS / stage) */
    int32_t stage_bytes;     /* (block_M*block_K + block_K*block_N) * 2; MXFP8:
                                (block_M + block_N) * (block_K + 4)               */
    int32_t lds_bytes;       /* lds_slots * stage_bytes (+ block_M * 128 with the chunked epilogue) */
    int64_t m_blocks, n_blocks, k_blocks, num_tiles;
    int32_t num_workgroups;  /* P; 0 while unresolved (default P before a device is seen) */
    int32_t waves;           /* waves of the busiest workgroup, ceil(ceil(m_blocks/cs) * n_blocks
                                / (P/cs)) for cluster size cs; 0 while P is unresolved        */
    int32_t threads_per_workgroup;
    int32_t xcd_remap;       /* 1: workgroup -> worker id permuted so XCDs get compact tile blocks */
    int32_t cluster_size;    /* tile scheduler: workgroups per cluster (1 = none)     */
    int32_t column_major;    /* tile scheduler: 1 = transposed tile walk              */
    int32_t store_block_N;   /* epilogue: 0 = direct stores, 64 = staged through LDS  */
    int32_t l2_prefetch;     /* 1: workers without a tile warm their XCD's L2 (tsgemm_set_l2_prefetch) */
} tsgemm_info;

/*
 * Validate a problem and build a plan.  Returns NULL on error (message in
 * tsgemm_last_error(), code in tsgemm_last_error_code()).  Makes no HIP call.
 * Defined by the host side of the persistent example (page "[Feature]
 * Introduce tile scheduler #2441", Files changed, gemm_persistent: m_blocks =
 * ceildiv(M, block_M), n_blocks = ceildiv(N, block_N), the worker count and
 * the K % block_K assertion) and by the argument checks of the lowered host
 * function (page "tilelang", section 1.3).
 *   M, N, K      >= 0; K % block_K == 0; N % 8 == 0 and K % 8 == 0 (16-byte rows,
 *                as the lowered host function's "divisible by 8" check);
 *                block_M*K*2, block_K*N*2 and block_M*N*2 below 2^31 (per-tile
 *                32-bit offsets); M, N < 2^31.
 *   dtype        TSGEMM_FP16 or TSGEMM_BF16 (A, B and C), or TSGEMM_MXFP8
 *                (see tsgemm_run_mx; 1-byte elements enter the 2^31 bounds).
 *   block_M/N/K  one of 128x128x32, 128x128x64, 256x256x32, 256x256x64;
 *                MXFP8: 256x256x128 only (K % 128 == 0, two LDS stages).
 *   group_size   >= 1, column blocks per rasterisation group.
 *   num_stages   >= 2: K-slabs in flight; the LDS ring holds
 *                min(num_stages, floor(160 KiB / stage_bytes), 5) of them.  A
 *                request deeper than that is not an error: the plan runs with
 *                the ring that fits and reports it as tsgemm_info.lds_slots
 *                (e.g. 256x256x64 tiles, 64 KiB a stage: 3 requested, 2 held).
 * The number of workgroups defaults to one per compute unit of the device
 * current at the first run (see tsgemm_set_num_workgroups).
 */
tsgemm_plan* tsgemm_create(int64_t M, int64_t N, int64_t K, int dtype,
                           int block_M, int block_N, int block_K,
                           int group_size, int num_stages);

/* Fix the persistent grid size P (>= 1); 0 restores "one per compute unit". */
int tsgemm_set_num_workgroups(tsgemm_plan* plan, int num_workgroups);

/* Wavefronts per workgroup: 4 (a 2x2 grid, one per SIMD) or 8 (2x4, two per
 * SIMD, so one wave's issue stalls leave the matrix core to the other); 0
 * restores the default for the tile shape.  Results are identical. */
int tsgemm_set_waves(tsgemm_plan* plan, int waves);

/* Tile scheduler options (page "[Feature] Introduce tile scheduler #2441",
 * the PR overview of PersistentTileScheduler and its 2-CTA example):
 *   cluster_size cs >= 1 (default 1): workgroup wid is rank wid % cs of
 *     cluster wid / cs; clusters walk a ceil(m_blocks/cs) x n_blocks grid of
 *     cluster tiles and each rank takes row block m*cs + rank, skipping the
 *     wave when that block is past the last row (the review's bounds guard).
 *     The number of workgroups must be a multiple of cs (checked at run).
 *   column_major (default 0): 1 walks row groups of group_size blocks, m
 *     fastest, instead of column groups with n fastest (the transpose).
 * Results of tsgemm_run do not depend on either option. */
int tsgemm_set_schedule(tsgemm_plan* plan, int column_major, int cluster_size);

/* Epilogue (page "[Feature] Introduce tile scheduler #2441", diff of the
 * persistent example: use_tma_store / store_block_N, the cast tile written to
 * shared memory and stored in column blocks).  store_block_N = 0 (default):
 * each lane stores its 16-byte pieces of C straight from registers; 64: the
 * tile leaves in 64-column chunks staged through an LDS buffer of block_M x 64
 * elements after the ring, every C row written as whole 128-byte segments.
 * The ring gives up a slot where both do not fit (tsgemm_info.lds_slots).
 * 4-wave kernels only (EUNSUPPORTED with 8 waves or MXFP8).  C is bit for bit
 * the same either way. */
int tsgemm_set_epilogue(tsgemm_plan* plan, int store_block_N);

/* Enable (1, default) or disable (0) the XCD-aware workgroup -> worker id
 * permutation.  The schedule is defined on worker ids either way. */
int tsgemm_set_xcd_remap(tsgemm_plan* plan, int enable);

/* With fewer tiles than workgroups, the workers that get no tile (the page's
 * persistent loop would end for them at once) instead warm the L2 of the XCD
 * they run on: they load one word of every 128-byte line of the A row panel
 * and B column panel that the XCD's active workers will stream, in K order,
 * and leave.  enable = 1 (default for fp16/bf16 plans) or 0 (they leave at
 * once).  The tile walk and C are the same either way; it shortens launches
 * whose inputs are not already in the Infinity Cache.  TSGEMM_EINVAL for
 * enable outside {0, 1}; TSGEMM_EUNSUPPORTED for enable = 1 on an MXFP8 plan. */
int tsgemm_set_l2_prefetch(tsgemm_plan* plan, int enable);

/* The workgroup -> worker id permutation a run uses (host only, no HIP call):
 * out[b] = worker id of workgroup b, for b < num_workgroups.  Workgroup b runs
 * on XCD b % num_xcds; each XCD gets contiguous runs of worker ids, and the
 * first num_active ids (the workers that have tiles: fewer than the
 * workgroups when the tiles run out) are split evenly over the XCDs.  A
 * permutation of [0, num_workgroups); TSGEMM_EINVAL unless num_workgroups,
 * num_xcds > 0 and 0 < num_active <= num_workgroups.  Not on the pages: the
 * renumbering is this implementation's (XCDs have separate L2 caches). */
int tsgemm_worker_numbering(int32_t num_workgroups, int32_t num_xcds, int32_t num_active, int32_t* out);

/* Asynchronously compute C = A*B on `stream` (a hipStream_t; NULL = default
 * stream).  The launch of page "tilelang" section 1.3 (call(A, B, C, stream):
 * one kernel on the caller's stream, 0 or an error code back); the product
 * and its persistent loop are those of page "[Feature] Introduce tile
 * scheduler #2441", Files changed, gemm_persistent (slabs of A and B staged
 * in shared memory, fp32 accumulation, cast and store per tile).  A, B, C: device pointers, 16-byte aligned, holding M*K, K*N and
 * M*N elements; C is fully overwritten and must not overlap A or B.  Buffers
 * must stay alive until the stream work completes.  M*N == 0 launches nothing. */
int tsgemm_run(const tsgemm_plan* plan, const void* A, const void* B, void* C, void* stream);

/* Same as tsgemm_run and additionally records every tile the GEMM kernel
 * processes: trace (DEVICE pointer, int32[4 * P * max_iters], max_iters =
 * tsgemm_info.waves for the run's P) receives (worker, iter, m_idx, n_idx) at
 * row worker*max_iters + iter.  Diagnostic; rows not visited are left untouched. */
int tsgemm_run_traced(const tsgemm_plan* plan, const void* A, const void* B, void* C,
                      void* stream, int32_t* trace);

/* Block-scaled FP8 (MX) product of a TSGEMM_MXFP8 plan, on `stream`:
 *
 *   C[m][n] = sum_k x(A[m][k]) * s(SFA[m][k/32]) * x(B[n][k]) * s(SFB[n][k/32])
 *
 * rounded once to bf16 (nearest, ties to even), fp32 accumulation.  The page
 * "[Feature] Introduce tile scheduler #2441" lists this MXFP8 block-scaled
 * persistent GEMM ("1d1d" scale factors SFA, SFB) among the examples driven
 * by the same tile scheduler, without its formats; they follow the OCP
 * Microscaling Formats specification v1.0:
 *   x(): FP8 E4M3 element (bias 7, subnormals, S.1111.111 = NaN, max 448);
 *   s(): E8M0 scale 2^(e - 127), 0xFF = NaN; one scale per 32 consecutive
 *        elements along K ("1d" blocks on both operands).
 * Layout (row-major, contiguous, DEVICE pointers, caller-owned):
 *   A   uint8[M][K]     B   uint8[N][K]   (both K-contiguous: B is given
 *   SFA uint8[M][K/32]  SFB uint8[N][K/32] transposed relative to tsgemm_run)
 *   C   bf16[M][N]
 * A, B, C 16-byte aligned, SFA and SFB 4-byte aligned.  Inner products are
 * formed by the gfx950 matrix core, which adds the up to 64 scaled products of
 * one instruction with an internal error (measured: at most about 2^-12 of
 * the sum of their magnitudes) before the fp32 accumulation, so C matches the
 * exact product to within that plus the final bf16 rounding, not bit for bit.  Scheduler
 * options, the number of workgroups and the XCD remap apply as for tsgemm_run;
 * tsgemm_set_waves accepts only 4.  M*N == 0 launches nothing; K == 0 gives
 * C = 0.  Returns TSGEMM_EINVAL for a plan of another dtype (and tsgemm_run
 * for an MXFP8 plan). */
int tsgemm_run_mx(const tsgemm_plan* plan, const void* A, const void* SFA, const void* B,
                  const void* SFB, void* C, void* stream);

/* tsgemm_run_mx plus the per-tile trace of tsgemm_run_traced. */
int tsgemm_run_mx_traced(const tsgemm_plan* plan, const void* A, const void* SFA, const void* B,
                         const void* SFB, void* C, void* stream, int32_t* trace);

/* Tile-blocked scale layout for tsgemm_run_mx_packed.  The row-major SFA/SFB
 * above make every lane of the kernel's scale fetch touch its own cache line
 * (one row each); the packed layout puts each tile's scales for a group of 4
 * slabs (512 elements of K) in one contiguous 4 KiB block:
 *   SFP[block][group][256][16]: block = 256-row block of A (operand 0) or of
 *   B's N rows (operand 1), group = g covers K blocks 16g .. 16g+15, row r of
 *   the block, byte j = SF[block*256 + r][16g + j]; rows past M (N) and bytes
 *   past K/32 are 0.
 * tsgemm_mx_packed_scale_bytes: bytes of SFP for `operand`
 *   (= blocks * ceil(k_blocks / 4) * 4096; 0 when K == 0), < 0 on error.
 * tsgemm_mx_pack_scales: writes SFP from SF (DEVICE pointers: SF 4-byte, SFP
 *   16-byte aligned, SFP holding tsgemm_mx_packed_scale_bytes bytes) on
 *   `stream`; a pure data permutation.
 * tsgemm_run_mx_packed: tsgemm_run_mx with packed SFA and SFB (16-byte
 *   aligned); C is bit for bit the result of tsgemm_run_mx on the unpacked
 *   scales.  For callers whose scale producer can write the packed layout, or
 *   who pack static (weight) scales once. */
int64_t tsgemm_mx_packed_scale_bytes(const tsgemm_plan* plan, int operand);
int tsgemm_mx_pack_scales(const tsgemm_plan* plan, int operand, const void* SF, void* SFP, void* stream);
int tsgemm_run_mx_packed(const tsgemm_plan* plan, const void* A, const void* SFAP, const void* B,
                         const void* SFBP, void* C, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * product of tsgemm_run_mx, computed as tsgemm_mx_pack_scales of SFA and of
 * SFB followed by tsgemm_run_mx_packed, with the packed scales kept in a
 * static workspace inside the library instead of caller buffers.  Same
 * arguments and result as tsgemm_run_mx (C bit for bit that of the packed
 * path).  Allocates nothing (no hipMalloc, no host allocation); the first call
 * on a device looks up the workspace's device address.
 *   Limit: packed SFA (rounded up to 256 bytes) + packed SFB at most 16 MiB,
 *   i.e. about (M + N) * K / 32 <= 16 MiB (8192^3: 4 MiB); larger plans get
 *   TSGEMM_EUNSUPPORTED before anything is launched.
 *   The workspace is one per device, held until the process ends, shared by
 *   every call on that device and left holding the last call's packed
 *   scales: calls that overlap on one device (different streams or threads
 *   without ordering between them) race on it. */
int tsgemm_run_mx_noalloc(const tsgemm_plan* plan, const void* A, const void* SFA, const void* B,
                          const void* SFB, void* C, void* stream);

/* m_blocks * n_blocks, the tile count the scheduler walks (page "[Feature]
 * Introduce tile scheduler #2441", Files changed: the waves formula
 * ceildiv(m_blocks * n_blocks, sm_num)); < 0 on error. */
int64_t tsgemm_num_tiles(const tsgemm_plan* plan);
int tsgemm_num_workgroups(const tsgemm_plan* plan);      /* resolves the default P      */
int tsgemm_plan_info(const tsgemm_plan* plan, tsgemm_info* info);

/* The launch geometry tsgemm_run would use on the current device: the number
 * of workgroups P (the explicit one, or one per compute unit), the waves of
 * the busiest worker (max_iters: a traced run writes P * max_iters rows) and
 * the XCD count the worker renumbering uses (1 when it is off).  Any output
 * pointer may be NULL.  Queries device attributes only for what the plan
 * leaves to the device (the default P; the XCD count when num_xcds is asked
 * for and the renumbering is on); launches nothing. */
int tsgemm_launch_info(const tsgemm_plan* plan, int32_t* num_workgroups, int32_t* max_iters,
                       int32_t* num_xcds);

/* Run the scheduler on the device over the plan's persistent grid and write
 * num_tiles rows of int32 (worker, iter, m_idx, n_idx), sorted by
 * (worker, iter), to the HOST buffer `out` (4 * num_tiles int32).
 * Synchronous (default stream); allocates and frees a device buffer of
 * 16 * P * max_iters bytes.  The scheduler is the one page "[Feature]
 * Introduce tile scheduler #2441" describes (Conversation tab, overview of
 * tile_schedule.py: init(worker), valid(), next_tile(), m_idx / n_idx and the
 * iteration counter current_iter; Files changed: the manual walk it replaces,
 * tile_id = sm_num * w + worker decoded in groups of group_size columns). */
int tsgemm_dump_schedule(const tsgemm_plan* plan, int32_t* out);

/* The same rows computed on the host by the same scheduler code compiled for
 * the CPU, for `num_workgroups` workers (> 0).  Makes no HIP call. */
int tsgemm_schedule_host(const tsgemm_plan* plan, int num_workgroups, int32_t* out);

/* Free a plan (host memory only; it holds no device resource).  NULL-safe.
 * The pages' host stubs (page "tilelang", section 1.3) keep their state in
 * statics and have no teardown; a plan here is an explicit object instead. */
void tsgemm_destroy(tsgemm_plan* plan);

/* Message of the last failing call on this thread ("" if none).  Valid until
 * the next tsgemm call on the same thread (page "tilelang", section 1.3:
 * get_last_error() returning the text kept by the failing call). */
const char* tsgemm_last_error(void);

/* TSGEMM_E* code of the last failing call on this thread (TSGEMM_OK if the
 * last call succeeded); for calls that return NULL rather than a code. */
int tsgemm_last_error_code(void);

#ifdef __cplusplus
}
#endif

#endif /* TSGEMM_H */
