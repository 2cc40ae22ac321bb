// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_rs.h"

namespace gemm_rs {

// Reduce work unit: kReduceRows output rows of one tile.
constexpr int kReduceRows = 32;
constexpr int kThreads = 256;

// Geometry the kernels need to place tiles.
struct TileGeom {
    int64_t M, N, K, Mc;
    int64_t slot;        // staging elements from slot (d,r) to the next (>= Mc*N)
    int32_t W, BM, BN, tiles_m, tiles_n, T, group_m, swizzle;
    int32_t interleave;  // q >= 1: tiles per destination visit (tile-interleaved order)
    int32_t bm_shift;    // log2(BM)
};

// Staging slot size in elements: Mc*N, rounded up to a multiple of
// 512 KiB once a slot holds 8 MiB or more.  A slot stride that is an odd
// multiple of 256 KiB (1000 rows of 8192 fp32, for one) was measured to
// cost the reduce's eight concurrent slot streams ~4% of their HBM rate;
// at 512 KiB multiples they run at the rate of power-of-two strides.  The
// rounding adds at most 1/16 to a slot.
__host__ __device__ inline int64_t staging_slot_elems(int64_t Mc, int64_t N, int elem_bytes) {
    const int64_t bytes = Mc * N * elem_bytes;
    const int64_t align = (int64_t)512 << 10;
    if (bytes < ((int64_t)8 << 20)) return Mc * N;
    return (bytes + align - 1) / align * align / elem_bytes;
}

// All tile-order arithmetic is 32-bit: b < W*T < 2^31 and d*Mc < M < 2^31
// (the plan rejects larger problems), and BM is a power of two.

// First tile-row whose first row lies in chunk d: ceil(d*Mc / BM), clipped.
__host__ __device__ inline int32_t chunk_first_tile_row(const TileGeom &g, int32_t d) {
    const uint32_t v = ((uint32_t)d * (uint32_t)g.Mc + (uint32_t)g.BM - 1u) >> g.bm_shift;
    return (int32_t)(v < (uint32_t)g.tiles_m ? v : (uint32_t)g.tiles_m);
}

__host__ __device__ inline int32_t dest_chunk(const TileGeom &g, int32_t r, int32_t s) {
    if (g.swizzle == GEMM_RS_SWIZZLE_REMOTE_FIRST ||
        g.swizzle == GEMM_RS_SWIZZLE_TILE_INTERLEAVED)
        return (r + 1 + s) % g.W;
    if (g.swizzle == GEMM_RS_SWIZZLE_SELF_FIRST) return (r + s) % g.W;
    return s;
}

// Tiles owned by chunk d: its tile-rows [first(d), first(d+1)) x tiles_n.
__host__ __device__ inline uint32_t chunk_tiles(const TileGeom &g, int32_t d) {
    return (uint32_t)(chunk_first_tile_row(g, d + 1) - chunk_first_tile_row(g, d)) *
           (uint32_t)g.tiles_n;
}

// The j-th tile of chunk d in its within-chunk order: tile-rows in groups
// of group_m, a group walked column by column, rows inside a column.
__host__ __device__ inline int32_t tile_in_chunk(const TileGeom &g, int32_t d, uint32_t j) {
    const uint32_t lo = (uint32_t)chunk_first_tile_row(g, d);
    const uint32_t rows = (uint32_t)chunk_first_tile_row(g, d + 1) - lo;
    const uint32_t gm = (uint32_t)g.group_m, tn_count = (uint32_t)g.tiles_n;
    const uint32_t per_group = gm * tn_count;
    const uint32_t grp = j / per_group;
    const uint32_t q = j - grp * per_group;
    const uint32_t left = rows - grp * gm;
    const uint32_t grp_rows = left < gm ? left : gm;
    const uint32_t tn = q / grp_rows;
    const uint32_t tm = lo + grp * gm + (q - tn * grp_rows);
    return (int32_t)(tm * tn_count + tn);
}

// Tile of workgroup b: rank r = b % W takes its k-th tile, k = b / W.
// Chunk-major orders: rank r walks destination chunks dest(r, 0..W-1), each
// chunk's tiles in their within-chunk order.  Tile-interleaved order: rank
// r visits dest(r, 0..W-1) in turn and takes the next q tiles of each on
// every visit (round j takes a chunk's tiles [j*q, (j+1)*q)), skipping
// used-up chunks.
__host__ __device__ inline void tile_of_block(const TileGeom &g, uint32_t b,
                                              int32_t *rank, int32_t *tile) {
    const uint32_t W = (uint32_t)g.W;
    const uint32_t r = b % W;
    uint32_t k = b / W;
    *rank = (int32_t)r;
    if (g.swizzle == GEMM_RS_SWIZZLE_TILE_INTERLEAVED) {
        // round j takes each destination's tiles [j*q, (j+1)*q), fewer
        // where a chunk runs out, in the visit order dest(r, 0..W-1)
        const uint32_t q = (uint32_t)g.interleave;
        uint32_t n_min = 0xffffffffu, n_max = 0;
        for (int32_t d = 0; d < g.W; ++d) {
            const uint32_t n = chunk_tiles(g, d);
            n_min = n < n_min ? n : n_min;
            n_max = n > n_max ? n : n_max;
        }
        const uint32_t full = n_min / q;   // rounds in which every chunk gives q tiles
        if (k < W * q * full) {
            const uint32_t j = k / (W * q), rem = k - j * (W * q);
            const uint32_t s = rem / q;
            *tile = tile_in_chunk(g, dest_chunk(g, (int32_t)r, (int32_t)s), j * q + (rem - s * q));
            return;
        }
        // tiles taken before round j: cb(j) = sum_d min(n_d, j*q); find the
        // last round j with cb(j) <= k (cb(full) <= k < cb(ceil(n_max/q)) = T)
        auto cb = [&](uint32_t jj) {
            uint32_t c = 0;
            for (int32_t d = 0; d < g.W; ++d) {
                const uint32_t n = chunk_tiles(g, d);
                c += n < jj * q ? n : jj * q;
            }
            return c;
        };
        uint32_t lo = full, hi = (n_max + q - 1) / q - 1;
        while (lo < hi) {
            const uint32_t mid = lo + (hi - lo + 1) / 2;
            if (cb(mid) <= k) lo = mid;
            else hi = mid - 1;
        }
        const uint32_t j = lo;
        uint32_t rem = k - cb(j);
        for (uint32_t s = 0; s < W; ++s) {
            const int32_t c = dest_chunk(g, (int32_t)r, (int32_t)s);
            const uint32_t n = chunk_tiles(g, c);
            const uint32_t left = n > j * q ? n - j * q : 0;
            const uint32_t avail = left < q ? left : q;
            if (rem < avail) {
                *tile = tile_in_chunk(g, c, j * q + rem);
                return;
            }
            rem -= avail;
        }
        *tile = 0;   // unreachable for k < T
        return;
    }
    for (int32_t s = 0; s < g.W; ++s) {
        const int32_t d = dest_chunk(g, (int32_t)r, s);
        const uint32_t n = chunk_tiles(g, d);
        if (k < n) {
            *tile = tile_in_chunk(g, d, k);
            return;
        }
        k -= n;
    }
    *tile = 0;   // unreachable for b < W*T
}

// Logical block of the h-th workgroup of a launch that covers logical
// blocks [b_offset, b_offset + n) (logical block k*W + r is rank r's k-th
// tile).  The hardware hands a launch's workgroups to the 8 XCDs round
// robin (h % 8).  When each rank's share of the launch, n/W tiles, splits
// evenly over the XCDs, XCD x takes the x-th eighth of every rank's part of
// the order, rank after rank: all XCDs then work on one rank's operands at a
// time, so the memory-side cache can serve that rank's B to every XCD after
// one read from HBM, while each XCD's L2 keeps its own tile-rows of A.
// Every rank's tile order is unchanged.  Otherwise the identity.  A
// bijection of [0, n) in both cases.
__host__ __device__ inline uint32_t logical_block(const TileGeom &g, uint32_t b_offset,
                                                  uint32_t n, uint32_t h) {
    constexpr uint32_t kXcds = 8;
    const uint32_t W = (uint32_t)g.W;
    if (b_offset % W != 0 || n % (kXcds * W) != 0) return b_offset + h;
    const uint32_t per = n / (kXcds * W);   // tiles of one rank per XCD
    const uint32_t x = h % kXcds, j = h / kXcds;
    const uint32_t r = j / per, k = x * per + j % per;
    return b_offset + k * W + r;
}

// Record the first asynchronous error of a run: {code, rank, tile, value}.
__device__ inline void record_error(int32_t *err, int code, int32_t r, int32_t t, uint32_t v) {
    if (atomicCAS(&err[0], 0, code) == 0) {
        __hip_atomic_store(&err[1], r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&err[2], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&err[3], (int32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Bounded wait until *f == 1 (0 = idle, 1 = ready, anything else breaks the
// protocol), with relaxed agent-scope loads: every waiter here runs after its
// producers' launch on the stream, whose boundary makes their stores
// visible.  Returns 0, or the error code after recording it.
__device__ inline int wait_flag_set(uint32_t *f, uint64_t timeout_ticks, int32_t *err,
                                    int32_t r, int32_t t) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
        const uint32_t v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v == 1u) return 0;
        if (v != 0u) {
            record_error(err, GEMM_RS_ERR_PROTOCOL, r, t, v);
            return GEMM_RS_ERR_PROTOCOL;
        }
        if (wall_clock64() - t0 > timeout_ticks) {
            record_error(err, GEMM_RS_ERR_TIMEOUT, r, t, 0);
            return GEMM_RS_ERR_TIMEOUT;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

enum { kFuseNone = 0, kFuseOwner = 1, kFuseLastArriver = 2 };

struct GemmArgs {
    TileGeom g;
    const void *A;       // [W][M][K]
    const void *B;       // [W][K][N]
    const void *C;       // nullable
    int64_t ldc;
    int32_t has_c;
    float alpha, beta;
    void *staging;       // [W][W] slots of g.slot elements ([Mc][N] used), float or bfloat16 bits
    int32_t staging_bf16;   // 1: stage partials as bfloat16 (round to nearest even)
    uint32_t *flags;     // [W][T]
    int32_t *trace;      // [W*T] or null
    int32_t release_flags;  // 1: the flag is read in this launch (last-arriver): it is
                            //    stored after a barrier and released with the count
    // 1: staging stores written through this XCD's L2 (`nt sc1` buffer
    // stores through one descriptor of staging_bytes < 4 GiB), so the
    // release before each flag finds no dirty staging lines to write back
    int32_t stage_wt;
    int64_t staging_bytes;
    // (rank << 26) | tile of every slot of the full launch (b_offset 0,
    // n_blocks W*T, the XCD map), tabulated once per plan; null: derive it
    // with logical_block and tile_of_block (launch slices, no plan)
    const uint32_t *slot_tab;
    uint32_t b_offset;      // first logical block of this launch (launch slices)
    uint32_t n_blocks;      // workgroups in this launch
    int32_t xcd_rank_major; // 1: logical_block's XCD map, 0: block = b_offset + blockIdx.x
    // all-gather mode (gemm_ag_*): tiles are stored as bfloat16 to
    // staging[r][row][col] (no chunk routing, flags == null), and a tile
    // first waits until signals[r*tiles_m + tm] == epoch, i.e. its rows of
    // A have arrived (bounded by timeout_ticks; a timeout is recorded in err)
    int32_t plain_out;
    const uint32_t *signals;
    // 1: the launch shares the CUs with another kernel's waves (the
    // identity-order reduce slices), so it keeps the register budget that
    // leaves them room (a gated all-gather launch, signals != null, too)
    int32_t coresident;
    uint32_t epoch;
    uint64_t timeout_ticks;
    int32_t *err;
    // reduce fused into the GEMM (kFuseOwner or kFuseLastArriver; 0 = none).
    // kFuseOwner (remote-first order, the launch of every rank's own-chunk
    // tiles): workgroup (rank r, tile t) is the last contribution to tile
    // t; it checks and resets the other ranks' flags for t, sums the
    // tile's W partials (the others from their staging slots, its own from
    // registers) in the reduce order and writes `out` (bf16).
    // kFuseLastArriver (one launch, any order): every producer stages its
    // partial, releases its flag and counts itself in on counters[t]; the
    // W-th sums the tile the same way.
    int32_t fuse_reduce;
    uint32_t *counters;     // [T] producer count per tile (kFuseLastArriver)
    int32_t keep_flags;     // kFuseLastArriver: leave the flags at 1
    int32_t groups;         // reduce order: G groups of W/G ranks (1: flat)
    void *out;              // [M][N]
};

enum { kSliceAll = 0, kSliceSteps = 2 };

struct ReduceArgs {
    TileGeom g;
    int32_t order, groups;   // groups == 1 for flat
    int32_t keep_flags;
    int32_t units_per_tile;  // BM / kReduceRows
    uint64_t timeout_ticks;  // device wall-clock ticks
    const void *staging;     // float, or bfloat16 bits (staging_bf16)
    int64_t staging_bytes;   // the whole staging (W*W slots)
    int32_t staging_bf16;
    void *out;               // [M][N]
    uint32_t *flags;         // [W][T]
    uint32_t *counters;      // [T] (flat) or [G][T] (sub stage)
    int32_t *err;            // {code, rank, tile, value}
    // which tiles the grid covers:
    //   kSliceAll      every tile
    //   kSliceSteps    the k-th tile of the common order for k in
    //                  [k_lo, k_hi) (identity order: every rank computes
    //                  tile seq[k] in step k)
    int32_t slice_kind;
    uint32_t k_lo, k_hi;
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
// Fill tab[h] = (rank << 26) | tile for the W*T slots of the full launch.
hipError_t launch_slot_table(const TileGeom &g, uint32_t *tab, hipStream_t s);
constexpr int kSlotTileBits = 26;
hipError_t launch_clear_words(uint32_t *a, int64_t na, uint32_t *b, int64_t nb,
                              hipStream_t s);

// Supported bf16 tile shapes (tile_m, tile_n).
bool bf16_tile_supported(int32_t bm, int32_t bn);
// Configurations that have an owner-fused reduce variant of the bf16 GEMM.
bool fused_reduce_supported(int32_t bm, int32_t bn, int32_t W);

}  // namespace gemm_rs
