/*
 * gemm_rs.h - fused GEMM + reduce-scatter epilogue + flag-gated reduce on
 * one MI355X (gfx950), with W virtual tensor-parallel ranks on one GPU.
 *
 * The operation (page "flux实现：sm80 gemm+rs", opening paragraph and
 * section "cutlass自定义epilogue–sm80"; page "flux精读", section 3 Design):
 * the second GEMM of an FFN block runs row-parallel over W ranks.  Rank r
 * holds A_r[M,K] and B_r[K,N]; its GEMM epilogue computes
 * alpha*acc + beta*C and, instead of writing an ordinary output, stores
 * every output tile straight into the reduce-scatter buffer slot of the
 * rank that will receive those rows.  Per-tile 32-bit ready flags tell the
 * reduce stage when a tile has landed (same page, StoreD paragraph: every
 * tile gets a unique id and only the producer/consumer relation is
 * tracked; page "flux精读", section 4.2: signals are contiguous 32-bit
 * words allocated once).  The reduce stage sums the W slots in a fixed
 * order, flat or two-level (page "flux实现：sm80 gemm+rs", section
 * "2D Ring优化"), and rank d receives rows [d*M/W, (d+1)*M/W) of
 *
 *     out = alpha * sum_r A_r B_r + beta * C
 *
 * with beta*C added once (by the rank that owns the row's chunk).
 *
 * Tile order: workgroup b of the W*T grid computes for rank b % W its
 * (b / W)-th tile; each rank visits remote chunks first and its own chunk
 * last, every rank starting at a different destination (page
 * "flux实现：sm80 gemm+rs", section "gemmrs版本的swizzle如何编排"; page
 * "通信 overlap 实现", Flux tile-fusion section).
 *
 * No pre-clear of any buffer is needed per run: each staging element has
 * exactly one writer per run and every flag the reduce consumes is put
 * back to 0 by the reduce itself (the clearing cost that page
 * "flux实现：sm80 gemm+rs", section "自己的类flux实现", measures is removed).
 *
 * All functions are plain C, never throw, never abort, never print.
 * Device pointers are HIP device addresses (for example a torch tensor's
 * data_ptr()); "stream" is a hipStream_t passed as void* (NULL = the
 * default stream).
 */
#ifndef GEMM_RS_H
#define GEMM_RS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_RS_API __attribute__((visibility("default")))

/* ---- status codes ------------------------------------------------------ */
#define GEMM_RS_OK            0
#define GEMM_RS_ERR_INVALID_ARG (-1) /* bad descriptor, pointer or flag     */
#define GEMM_RS_ERR_UNSUPPORTED (-2) /* valid problem, not implemented      */
#define GEMM_RS_ERR_HIP       (-3)  /* a HIP call failed (alloc / launch)    */
#define GEMM_RS_ERR_TIMEOUT   (-4)  /* async: a flag wait ran out of time    */
#define GEMM_RS_ERR_PROTOCOL  (-5)  /* async: a flag held neither 0 nor 1    */
#define GEMM_RS_ERR_SCRATCH   (-6)  /* gemm_rs_run_noalloc: the workspace
                                       exceeds its static scratch          */

/* ---- descriptor enums -------------------------------------------------- */
#define GEMM_RS_BF16 0 /* A, B, C bfloat16; out bfloat16 (RNE); fp32 accumulate */
#define GEMM_RS_F32  1 /* A, B, C, out float32                                */

#define GEMM_RS_ORDER_FLAT      0 /* y = ((S_0 + S_1) + ...) + S_{W-1}        */
#define GEMM_RS_ORDER_TWO_LEVEL 1 /* groups of W/G ranks, then across groups  */

#define GEMM_RS_SWIZZLE_REMOTE_FIRST 0 /* dest(r,s) = (r+1+s) mod W (default) */
#define GEMM_RS_SWIZZLE_SELF_FIRST   1 /* dest(r,s) = (r+s) mod W             */
#define GEMM_RS_SWIZZLE_IDENTITY     2 /* dest(r,s) = s (no swizzle)          */
#define GEMM_RS_SWIZZLE_TILE_INTERLEAVED 3 /* dest(r,s) = (r+1+s) mod W, visited
                                              q = interleave tiles at a time:
                                              rank r's k-th tile goes to
                                              dest(r, (k/q) mod W) while every
                                              chunk has tiles left */

/* staging element type (gemm_rs_desc_t.staging_dtype) */
#define GEMM_RS_STAGING_F32  0
#define GEMM_RS_STAGING_BF16 1

/* ---- run flags ---------------------------------------------------------- */
#define GEMM_RS_RUN_GEMM    1u /* GEMM + epilogue + flag publish            */
#define GEMM_RS_RUN_REDUCE  2u /* flag-gated reduce (+ flag reset)          */
#define GEMM_RS_KEEP_FLAGS  4u /* debug: the reduce leaves flags at 1       */
#define GEMM_RS_TRACE_TILES 8u /* debug: GEMM records trace[b] = tile of WG b */
#define GEMM_RS_OVERLAP_REDUCE 16u /* with RUN_GEMM|RUN_REDUCE: take the reduce
                                      off the serial path (owner-fused or
                                      overlapped; see gemm_rs_run) */
#define GEMM_RS_LAST_ARRIVER 32u /* with RUN_GEMM|RUN_REDUCE: one launch, each
                                    tile summed by its last producer (see
                                    gemm_rs_run) */
#define GEMM_RS_RUN_ALL     (GEMM_RS_RUN_GEMM | GEMM_RS_RUN_REDUCE)

/*
 * Problem descriptor.  Shapes follow the pages' problem statement: W ranks,
 * per-rank A_r[M,K] and B_r[K,N], alpha, beta, optional C, tile shape, and
 * a flat or two-level reduction order.
 *
 *   M, N, K      per-rank GEMM shape; M % W == 0 (rank d receives M/W rows);
 *                each below 2^31; M, N >= 1.  K == 0 is allowed: the
 *                empty sum, so every partial is 0 and out = beta*C
 *                (A and B are then never read and may be NULL)
 *   W            virtual ranks, 1..64
 *   dtype        GEMM_RS_BF16 or GEMM_RS_F32
 *   tile_m/_n    output tile (the communication unit); 0 picks a default.
 *                bf16: 256x256, 256x128, 128x128, 64x128; f32: 64x64.
 *   group_m      tile-rows per group inside a chunk; 1: row-major;
 *                0: the default, 4
 *   order        GEMM_RS_ORDER_*; groups = G for the two-level order
 *                (W % G == 0; ranks g*W/G .. (g+1)*W/G-1 form group g)
 *   swizzle      GEMM_RS_SWIZZLE_*
 *   has_c, ldc   C present; ldc = 0: C is one row of N broadcast to every
 *                row; ldc >= N: C is [M][ldc] row-major.  ldc % 8 == 0.
 *   materialize_sub  two-level only: write each group's partial sum to a
 *                sub-group buffer with its own flags before the final sum
 *   timeout_ms   bound on every device flag wait; 0 = 1000 ms
 *   staging_dtype  GEMM_RS_STAGING_F32 (default): partials are staged in
 *                float32, the precision the fixed-order reduce sums in.
 *                GEMM_RS_STAGING_BF16 (bf16 inputs only, not with
 *                materialize_sub): each partial is rounded to bfloat16
 *                (nearest even) when staged, halving the staging traffic
 *                of both kernels at the cost of a second rounding per
 *                partial; the reduce still sums in float32 in fixed order.
 *   interleave   tiles per destination visit of GEMM_RS_SWIZZLE_TILE_INTERLEAVED
 *                (round j takes each destination's tiles [j*q, (j+1)*q));
 *                0 or 1: one tile per visit; more than 1 with another
 *                swizzle is INVALID_ARG.  A q of at least a chunk's tile
 *                count gives the chunk-major remote-first order.
 */
typedef struct gemm_rs_desc {
    int64_t M, N, K;
    int32_t W;
    int32_t dtype;
    int32_t tile_m, tile_n;
    int32_t group_m;
    int32_t order;
    int32_t groups;
    int32_t swizzle;
    int32_t has_c;
    int32_t materialize_sub;
    int64_t ldc;
    uint32_t timeout_ms;
    uint32_t staging_dtype;
    int32_t interleave;
} gemm_rs_desc_t;

typedef struct gemm_rs_plan_s *gemm_rs_plan_t;

/*
 * Introspection record (tests and benchmark).  Workspace pointers are
 * device addresses owned by the plan.
 *   staging      W*W slots S[d][r] of slot_elems elements (float32, or
 *                bfloat16 bits with GEMM_RS_STAGING_BF16): slot (d,r) at
 *                element (d*W + r)*slot_elems holds [Mc][N] row-major;
 *                slot_elems = Mc*N, rounded up to a multiple of 512 KiB
 *                when a slot holds 8 MiB or more (the rest of the slot is
 *                never read or written)
 *   flags        uint32 flag[r][t], r < W, t < T (t = tm*tiles_n + tn)
 *   sub          float32 sub[d][g][Mc][N] (materialize_sub only, else NULL)
 *   sub_flags    uint32 subflag[g][t] (materialize_sub only, else NULL)
 *   trace        int32 trace[b], b < W*T (written under GEMM_RS_TRACE_TILES)
 */
typedef struct gemm_rs_info {
    int64_t Mc;
    int32_t tile_m, tile_n;
    int32_t tiles_m, tiles_n, T;
    int32_t group_m;
    int64_t workspace_bytes;
    void *staging;
    void *flags;
    void *sub;
    void *sub_flags;
    void *trace;
    int64_t staging_bytes, flags_bytes, sub_bytes, sub_flags_bytes;
    int64_t slot_elems;
} gemm_rs_info_t;

/*
 * gemm_rs_plan: validate *desc, choose defaults, allocate the workspace on
 * the current HIP device (staging W*W*slot_elems elements, flags, counters, error
 * word, trace, optional sub-group buffers) and zero the flags once,
 * synchronously.  On success *out owns all of it until gemm_rs_destroy.
 * Returns OK, INVALID_ARG (NULL desc/out, W outside 1..64, M or N < 1,
 * K < 0, M % W != 0,
 * unknown enum, bad ldc, materialize_sub without the two-level order),
 * UNSUPPORTED (tile not in the set above, N % tile_n != 0, K % 64 != 0,
 * ldc % 8 != 0, M, N or K of 2^31 or more, bf16 with K of 2^23 or more or
 * N of 2^25 or more (32-bit offsets in one K step's operand windows), grid
 * over 2^31-1) or HIP.  Invalid descriptors are
 * rejected before any HIP call.  On failure *out is set to NULL.
 */
GEMM_RS_API int gemm_rs_plan(const gemm_rs_desc_t *desc, gemm_rs_plan_t *out);

/*
 * Device: a plan belongs to the device that was current at gemm_rs_plan.
 * gemm_rs_run, gemm_rs_tile_order and gemm_rs_status must be called with
 * that device current (they return INVALID_ARG otherwise, before enqueuing
 * anything); gemm_rs_destroy switches to it by itself.
 */

/*
 * gemm_rs_run: enqueue one pass on `stream`, with no host synchronisation
 * and no memset.
 *   A    [W][M][K] row-major (dtype), 16-byte aligned     (RUN_GEMM)
 *   B    [W][K][N] row-major (dtype), 16-byte aligned     (RUN_GEMM)
 *   C    see desc.has_c; NULL when has_c == 0             (RUN_GEMM)
 *   out  [M][N] row-major (dtype), 16-byte aligned        (RUN_REDUCE);
 *        rows [d*M/W, (d+1)*M/W) are rank d's chunk
 *   run_flags  GEMM_RS_RUN_GEMM | GEMM_RS_RUN_REDUCE, plus the debug bits,
 *              plus GEMM_RS_OVERLAP_REDUCE
 * GEMM_RS_OVERLAP_REDUCE (both RUN bits, flat or register two-level
 * reduce, every chunk owning the same number of tile rows; otherwise
 * ignored) takes the reduce off the serial path in one of two ways:
 *   - remote-first tile order (owner-fused reduce; bf16, 256x256 tiles,
 *     W = 8, without KEEP_FLAGS, else the serial path): every rank visits
 *     its own chunk last, so rank d's last step is the last contribution
 *     to every tile of chunk d, and the other ranks' partials of those
 *     tiles come from earlier steps.  The earlier steps run as one launch;
 *     in a second launch on `stream` each of rank d's last-step workgroups
 *     checks and resets the other ranks' flags for its tile, sums the
 *     tile's W partials in the reduce order (its own from registers, never
 *     staged) and writes its rows of `out`.  No separate reduce runs.
 *   - identity tile order: every rank computes chunk c in the same steps;
 *     the GEMM is launched chunk group by chunk group (up to eight) and,
 *     after each, an auxiliary stream owned by the plan reduces the chunks
 *     it completed, concurrently with the next group; `stream` waits for
 *     the auxiliary stream at the end.
 * GEMM_RS_LAST_ARRIVER (both RUN bits; bf16, 256x256 tiles, W = 8, flat or
 * register two-level reduce; not with OVERLAP_REDUCE, which is
 * INVALID_ARG; otherwise the serial path): the whole pass is one GEMM
 * launch in any tile order.  Every producer stages its partial (fp32
 * staging below 4 GiB is written through its XCD's L2), sets its tile
 * flag, and then counts itself in on the tile's counter with a relaxed
 * agent-scope add behind an agent-scope release fence, which orders the
 * staged partial and the flag before the count.  The producer that
 * completes the count (page "flux实现：sm80 gemm+rs", section "device side
 * barrier": the counter whose last arrival ends the wait) takes an
 * agent-scope acquire, checks and resets the tile's flags and counter and
 * sums the tile's W partials in the reduce order (its own from registers)
 * into `out`.  No workgroup waits for another, so it cannot deadlock
 * whatever the residency; each producer pays the release.
 * Results are bit-identical to the serial order.
 * The caller owns A, B, C, out and the stream, and keeps them alive until
 * the stream's work is done.  Calls on one stream are ordered; one plan
 * must not run on two streams at once.  A device-side flag-wait timeout or
 * protocol error does not fail this call: the kernel records it and
 * exits, and gemm_rs_status reports it.  Returns OK, INVALID_ARG or HIP.
 */
GEMM_RS_API int gemm_rs_run(gemm_rs_plan_t plan, const void *A, const void *B,
                const void *C, float alpha, float beta, void *out,
                void *stream, uint32_t run_flags);

/*
 * gemm_rs_run_noalloc: gemm_rs_run without a plan and without allocating,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * validates *desc as gemm_rs_plan does and enqueues one whole pass on
 * `stream` with the same kernels, keeping the workspace (error record,
 * flags, counters, staging) in one static device array of 64 MiB per GPU,
 * held from the library's first use on that GPU until the process ends.
 * No hipMalloc, hipFree, stream or event creation, and no host
 * synchronisation.
 *   desc, A, B, C, alpha, beta, out, stream: as for gemm_rs_plan and
 *        gemm_rs_run (pointers are caller-owned device memory)
 *   run_flags  GEMM_RS_RUN_ALL, optionally | GEMM_RS_OVERLAP_REDUCE (the
 *        owner-fused reduce where gemm_rs_run would use it; the identity
 *        order's second-stream overlap runs serially here) or
 *        | GEMM_RS_LAST_ARRIVER.  Split passes
 *        and the debug bits are INVALID_ARG: the flags are cleared at the
 *        start of every call.
 *   status  NULL, or 4 int32 of 16-byte-aligned device memory: zeroed at
 *        the start of the pass, then {code, rank, tile, value} of the first
 *        asynchronous error (TIMEOUT or PROTOCOL) of the pass
 * Returns OK, INVALID_ARG / UNSUPPORTED (as gemm_rs_plan; materialize_sub
 * is UNSUPPORTED here), SCRATCH when the workspace (256 bytes + W*T*4 +
 * T*4, each rounded up to 256, + W*W*slot_elems staging elements of 4
 * bytes, 2 with bfloat16 staging; see gemm_rs_info_t) exceeds 64 MiB, or
 * HIP.  Every call on one GPU shares the same
 * array: calls that overlap on one GPU (two streams, or two threads) race
 * and give undefined results; calls ordered on one stream are safe.
 */
GEMM_RS_API int gemm_rs_run_noalloc(const gemm_rs_desc_t *desc, const void *A,
                                    const void *B, const void *C, float alpha,
                                    float beta, void *out, void *stream,
                                    uint32_t run_flags, int32_t *status);

/*
 * gemm_rs_destroy: free the workspace.  The caller must synchronise every
 * stream that used the plan first.  destroy(NULL) returns OK.
 */
GEMM_RS_API int gemm_rs_destroy(gemm_rs_plan_t plan);

/* gemm_rs_query: fill *info.  Returns OK or INVALID_ARG. */
GEMM_RS_API int gemm_rs_query(gemm_rs_plan_t plan, gemm_rs_info_t *info);

/*
 * gemm_rs_tile_order: evaluate on the device, with the same device
 * function the GEMM kernel uses, the tile of every workgroup b < W*T and
 * copy it to host_trace[W*T] (host memory).  Synchronous.
 */
GEMM_RS_API int gemm_rs_tile_order(gemm_rs_plan_t plan, int32_t *host_trace);

/*
 * gemm_rs_status: synchronise `stream`, return the first asynchronous
 * error recorded by a kernel since the last call (OK, TIMEOUT or
 * PROTOCOL), write {code, rank, tile, value} to detail[4] when detail is
 * not NULL, clear the record and, after an error, put every flag and
 * counter back to 0 so the plan can run again.  Returns HIP if a HIP call
 * fails.
 */
GEMM_RS_API int gemm_rs_status(gemm_rs_plan_t plan, void *stream, int32_t *detail);

/* gemm_rs_strerror: static text for a status code. */
GEMM_RS_API const char *gemm_rs_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_RS_H */
