// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_rs.h"

namespace gemm_rs {

// Reduce work unit: kReduceRows output rows of one tile.
#ifndef GEMM_RS_REDUCE_ROWS
#define GEMM_RS_REDUCE_ROWS 32
#endif
constexpr int kReduceRows = GEMM_RS_REDUCE_ROWS;
constexpr int kThreads = 256;

// Geometry the kernels need to place tiles.
struct TileGeom {
    int64_t M, N, K, Mc;
    int32_t W, BM, BN, tiles_m, tiles_n, T, group_m, swizzle;
};

// First tile-row whose first row lies in chunk d: ceil(d*Mc / BM), clipped.
__host__ __device__ inline int32_t chunk_first_tile_row(const TileGeom &g, int32_t d) {
    int64_t v = ((int64_t)d * g.Mc + g.BM - 1) / g.BM;
    return (int32_t)(v < g.tiles_m ? v : g.tiles_m);
}

__host__ __device__ inline int32_t dest_chunk(const TileGeom &g, int32_t r, int32_t s) {
    if (g.swizzle == GEMM_RS_SWIZZLE_REMOTE_FIRST) return (r + 1 + s) % g.W;
    if (g.swizzle == GEMM_RS_SWIZZLE_SELF_FIRST) return (r + s) % g.W;
    return s;
}

// Tile of workgroup b: rank r = b % W takes its k-th tile, k = b / W.
// Rank r walks destination chunks dest(r, 0..W-1); chunk d holds the
// tile-rows [first(d), first(d+1)); inside a chunk, tile-rows are grouped
// by group_m and a group is walked column by column, rows inside a column.
__host__ __device__ inline void tile_of_block(const TileGeom &g, int64_t b,
                                              int32_t *rank, int32_t *tile) {
    const int32_t r = (int32_t)(b % g.W);
    int64_t k = b / g.W;
    int32_t tm = 0, tn = 0;
    for (int32_t s = 0; s < g.W; ++s) {
        const int32_t d = dest_chunk(g, r, s);
        const int32_t lo = chunk_first_tile_row(g, d);
        const int32_t rows = chunk_first_tile_row(g, d + 1) - lo;
        const int64_t n = (int64_t)rows * g.tiles_n;
        if (k < n) {
            const int32_t gm = g.group_m;
            const int64_t per_group = (int64_t)gm * g.tiles_n;
            const int32_t grp = (int32_t)(k / per_group);
            const int32_t q = (int32_t)(k - (int64_t)grp * per_group);
            const int32_t grp_rows = (rows - grp * gm) < gm ? (rows - grp * gm) : gm;
            tn = q / grp_rows;
            tm = lo + grp * gm + q % grp_rows;
            break;
        }
        k -= n;
    }
    *rank = r;
    *tile = tm * g.tiles_n + tn;
}

struct GemmArgs {
    TileGeom g;
    const void *A;       // [W][M][K]
    const void *B;       // [W][K][N]
    const void *C;       // nullable
    int64_t ldc;
    int32_t has_c;
    float alpha, beta;
    float *staging;      // [W][W][Mc][N]
    uint32_t *flags;     // [W][T]
    int32_t *trace;      // [W*T] or null
    int32_t release_flags;  // 1: agent-scope release (concurrent consumer)
};

struct ReduceArgs {
    TileGeom g;
    int32_t order, groups;   // groups == 1 for flat
    int32_t keep_flags;
    int32_t acquire;         // 1: producers may run concurrently
    int32_t units_per_tile;  // BM / kReduceRows
    uint64_t timeout_ticks;  // device wall-clock ticks
    const float *staging;
    void *out;               // [M][N]
    uint32_t *flags;         // [W][T]
    uint32_t *counters;      // [T] (flat) or [G][T] (sub stage)
    int32_t *err;            // {code, rank, tile, value}
    // materialised two-level buffers (sub stage writes, final stage reads)
    float *sub;              // [W][G][Mc][N]
    uint32_t *sub_flags;     // [G][T*units_per_tile]
};

// Launchers (return hipError_t of the launch).
hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs &a, int dtype, hipStream_t s);
hipError_t launch_reduce_sub(const ReduceArgs &a, hipStream_t s);
hipError_t launch_reduce_final_sub(const ReduceArgs &a, int dtype, hipStream_t s);
hipError_t launch_tile_order(const TileGeom &g, int32_t *trace, hipStream_t s);

// Supported bf16 tile shapes (tile_m, tile_n).
bool bf16_tile_supported(int32_t bm, int32_t bn);

}  // namespace gemm_rs
