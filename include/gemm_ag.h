/*
 * gemm_ag.h - all-gather fused into the prologue of a GEMM, on one AMD
 * Instinct MI355X (gfx950), W virtual tensor-parallel ranks.
 *
 * The other half of the Flux design (page "flux精读", section 3 Design and
 * section 4.2 Implementation details; page "通信 overlap 实现", Flux
 * tile-fusion section, AG+GEMM bullet): the input X is sharded by rows
 * across the W ranks (rank d holds rows [d*M/W, (d+1)*M/W)); every rank
 * needs all of X for its GEMM Y_r = X . B_r.  Instead of gathering X and
 * then multiplying, the gather is issued as copies tile by tile, each
 * finished tile sets a 32-bit signal, and each GEMM workgroup waits for the
 * signal of the tile-row of X it needs before its mainloop starts, in the
 * order the tiles are sent.
 *
 * On one GPU: rank r's gathered X is a buffer the plan owns; a copy kernel
 * on a second stream stands in for the DMA transfers (one tile-row of X per
 * signal, each rank's own chunk first, then the following chunks), and
 * publishes signal[r][tm] = epoch with an agent-scope release; the GEMM
 * (the bf16 kernel of gemm_rs.h) gates each tile on an agent-scope acquire
 * of that signal.  Signals carry a per-run epoch, so they are never reset.
 * A wait is bounded; a timeout is reported, never a hang.
 *
 * Shares the status codes of gemm_rs.h (GEMM_RS_OK, ..._INVALID_ARG,
 * ..._UNSUPPORTED, ..._HIP, ..._TIMEOUT) and gemm_rs_strerror.
 */
#ifndef GEMM_AG_H
#define GEMM_AG_H

#include <stdint.h>

#include "gemm_rs.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---- run flags ---------------------------------------------------------- */
#define GEMM_AG_RUN_COPY   1u /* gather X into every rank's buffer, publish signals */
#define GEMM_AG_RUN_GEMM   2u /* the gated GEMM, Y_r = X_gathered_r . B_r            */
#define GEMM_AG_FUSED      4u /* with both: copies on the plan's second stream,
                                 concurrent with the GEMM on `stream` (tiles wait
                                 for their signals); without it: copies, then the
                                 GEMM, in order on `stream`                        */
#define GEMM_AG_EXPECT_NEXT 8u /* debug, RUN_GEMM alone: wait for the next epoch,
                                  which no copy publishes (forces the timeout path) */
#define GEMM_AG_RUN_ALL    (GEMM_AG_RUN_COPY | GEMM_AG_RUN_GEMM)

/*
 * Problem descriptor.
 *   M, N, K      per-rank GEMM Y_r[M,N] = X[M,K] . B_r[K,N]; M % W == 0 (rank
 *                d holds rows [d*M/W, (d+1)*M/W) of X); each below 2^31
 *   W            virtual ranks, 1..64
 *   tile_m/_n    output tile, 0 picks the default; bf16 tiles as in gemm_rs.h
 *   group_m      tile-rows per group in the tile order; 0: 4
 *   timeout_ms   bound on every signal wait; 0 = 1000 ms
 *   pad          must be 0
 * The communication tile is one tile-row of X (tile_m rows x K).
 */
typedef struct gemm_ag_desc {
    int64_t M, N, K;
    int32_t W;
    int32_t tile_m, tile_n;
    int32_t group_m;
    uint32_t timeout_ms;
    uint32_t pad;
} gemm_ag_desc_t;

typedef struct gemm_ag_plan_s *gemm_ag_plan_t;

/*
 * Introspection record.  Device addresses owned by the plan:
 *   gathered     bfloat16 X_r[W][M][K]: rank r's copy of the gathered X
 *   signals      uint32 signal[W][tiles_m], equal to `epoch` once the tile-row
 *                has been copied in the latest run with RUN_COPY
 */
typedef struct gemm_ag_info {
    int32_t tile_m, tile_n;
    int32_t tiles_m, tiles_n;
    int32_t group_m;
    uint32_t epoch;
    void *gathered;
    void *signals;
    int64_t gathered_bytes;
} gemm_ag_info_t;

/*
 * gemm_ag_plan: validate, allocate the gathered buffers, signals, error
 * word and the second stream, zero the signals (synchronously).
 * Returns OK, INVALID_ARG (NULL pointers, W, M % W, pad != 0, ...),
 * UNSUPPORTED (tile, N % tile_n, K % 64, sizes: each below 2^31, K below
 * 2^23 and N below 2^25) or HIP.
 */
GEMM_RS_API int gemm_ag_plan(const gemm_ag_desc_t *desc, gemm_ag_plan_t *out_plan);

/*
 * Device: a plan belongs to the device that was current at gemm_ag_plan;
 * gemm_ag_run and gemm_ag_status return INVALID_ARG unless that device is
 * current; gemm_ag_destroy switches to it by itself.
 */

/*
 * gemm_ag_run: enqueue one pass on `stream`, no host synchronisation.
 *   X    [W][M/W][K] bfloat16 row shards, 16-byte aligned     (RUN_COPY)
 *   B    [W][K][N]   bfloat16, row-major, 16-byte aligned     (RUN_GEMM)
 *   out  [W][M][N]   bfloat16, rank r's Y_r at out + r*M*N    (RUN_GEMM)
 * RUN_COPY advances the plan's epoch.  RUN_GEMM alone uses the gathered
 * buffers of the latest copy (its signals already hold the epoch).  A
 * signal-wait timeout does not fail this call: the kernel records it and
 * exits, and gemm_ag_status reports it.  The caller keeps X, B, out and
 * the stream alive until the work is done; one plan runs on one stream at
 * a time.  Returns OK, INVALID_ARG or HIP.
 */
GEMM_RS_API int gemm_ag_run(gemm_ag_plan_t plan, const void *X, const void *B, void *out,
                            void *stream, uint32_t run_flags);

/* gemm_ag_query: fill *info.  OK or INVALID_ARG. */
GEMM_RS_API int gemm_ag_query(gemm_ag_plan_t plan, gemm_ag_info_t *info);

/*
 * gemm_ag_status: synchronise `stream` and the plan's second stream, return
 * the first recorded device error (OK, TIMEOUT) with detail {code, rank,
 * tile-row, 0}, and clear it.  A timed-out run leaves its outputs undefined.
 */
GEMM_RS_API int gemm_ag_status(gemm_ag_plan_t plan, void *stream, int32_t *detail4);

/* gemm_ag_destroy: free the workspace (synchronise first).  NULL is OK. */
GEMM_RS_API int gemm_ag_destroy(gemm_ag_plan_t plan);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_AG_H */
