// Host side of the C ABI: descriptor validation, workspace ownership and
// kernel launch sequencing.  No host synchronisation and no memset on the
// run path.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "gemm_rs.h"
#include "gemm_rs_internal.h"

using namespace gemm_rs;

// Workspace of gemm_rs_run_noalloc (see device_scratch below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// overlapped reduce with the identity order: at most this many chunk groups
constexpr int kChunkSlices = 8;
constexpr int kEvents = kChunkSlices;

struct gemm_rs_plan_s {
    gemm_rs_desc_t d;        // resolved (tiles, group_m, timeout filled in)
    TileGeom g;
    int device;
    int32_t units_per_tile;
    uint64_t timeout_ticks;
    void *staging;           // float or bfloat16 bits (staging_dtype)
    uint32_t *flags;         // [W][T]
    uint32_t *counters;      // [T]
    uint32_t *sub_counters;  // [G][T] (materialised two-level)
    float *sub;              // [W][G][Mc][N]
    uint32_t *sub_flags;     // [G][T*units]
    int32_t *err;            // 4 words
    int32_t *trace;          // [W*T]
    uint32_t *slot_tab;      // [W*T] (rank, tile) of each slot of the full launch, or null
    int64_t staging_bytes, flags_bytes, counters_bytes, sub_bytes,
        sub_flags_bytes, trace_bytes;
    // overlapped reduce: an auxiliary stream (default priority) and events
    hipStream_t aux;
    hipEvent_t slice_done[kEvents];
    hipEvent_t aux_done;
    bool uniform_chunks;     // every chunk owns the same number of tiles
};

namespace {

constexpr int kMaxW = 64;
constexpr int kKStep = 64;
constexpr int64_t kMaxKBf16 = int64_t(1) << 23;
constexpr int64_t kMaxNBf16 = int64_t(1) << 25;

bool f32_tile_supported(int32_t bm, int32_t bn) { return bm == 64 && bn == 64; }

// Default tile: the largest supported tile that the shape fills.
void pick_default_tile(const gemm_rs_desc_t &d, int32_t *bm, int32_t *bn) {
    if (d.dtype == GEMM_RS_F32) {
        *bm = d.tile_m ? d.tile_m : 64;
        *bn = d.tile_n ? d.tile_n : 64;
        return;
    }
    int32_t m = d.tile_m, n = d.tile_n;
    if (m == 0) m = (d.M <= 64) ? 64 : 256;
    if (n == 0) {
        if (m == 64) n = 128;
        else n = (d.N % 256 == 0) ? 256 : 128;
    }
    *bm = m;
    *bn = n;
}

// Problem-level checks: INVALID_ARG.  Implementation limits: UNSUPPORTED.
int validate(const gemm_rs_desc_t &d, int32_t bm, int32_t bn) {
    // K == 0 is the empty sum: every partial is 0 and out = beta*C
    if (d.W < 1 || d.W > kMaxW || d.M < 1 || d.N < 1 || d.K < 0)
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.M % d.W != 0) return GEMM_RS_ERR_INVALID_ARG;
    if (d.dtype != GEMM_RS_BF16 && d.dtype != GEMM_RS_F32)
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.group_m < 0 || d.tile_m < 0 || d.tile_n < 0)
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.order != GEMM_RS_ORDER_FLAT && d.order != GEMM_RS_ORDER_TWO_LEVEL)
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.order == GEMM_RS_ORDER_TWO_LEVEL &&
        (d.groups < 1 || d.W % d.groups != 0))
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.swizzle != GEMM_RS_SWIZZLE_REMOTE_FIRST &&
        d.swizzle != GEMM_RS_SWIZZLE_SELF_FIRST &&
        d.swizzle != GEMM_RS_SWIZZLE_IDENTITY &&
        d.swizzle != GEMM_RS_SWIZZLE_TILE_INTERLEAVED)
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.interleave < 0 || (d.interleave > 1 && d.swizzle != GEMM_RS_SWIZZLE_TILE_INTERLEAVED))
        return GEMM_RS_ERR_INVALID_ARG;
    if ((d.has_c != 0 && d.has_c != 1) || d.ldc < 0 ||
        (d.has_c && d.ldc != 0 && d.ldc < d.N))
        return GEMM_RS_ERR_INVALID_ARG;
    if ((d.materialize_sub != 0 && d.materialize_sub != 1) ||
        (d.materialize_sub && d.order != GEMM_RS_ORDER_TWO_LEVEL))
        return GEMM_RS_ERR_INVALID_ARG;
    if (d.staging_dtype != GEMM_RS_STAGING_F32 && d.staging_dtype != GEMM_RS_STAGING_BF16)
        return GEMM_RS_ERR_INVALID_ARG;
    bool tile_ok = d.dtype == GEMM_RS_BF16 ? bf16_tile_supported(bm, bn)
                                           : f32_tile_supported(bm, bn);
    if (!tile_ok) return GEMM_RS_ERR_UNSUPPORTED;
    if (d.N % bn != 0 || d.K % kKStep != 0) return GEMM_RS_ERR_UNSUPPORTED;
    if (d.has_c && d.ldc % 8 != 0) return GEMM_RS_ERR_UNSUPPORTED;
    if (d.staging_dtype == GEMM_RS_STAGING_BF16 &&
        (d.dtype != GEMM_RS_BF16 || d.materialize_sub))
        return GEMM_RS_ERR_UNSUPPORTED;
    if (d.M > INT32_MAX || d.N > INT32_MAX || d.K > INT32_MAX)
        return GEMM_RS_ERR_UNSUPPORTED;
    // the bf16 kernel addresses one K step's A and B windows with 32-bit
    // buffer offsets: up to 256 rows of K and 64 rows of N elements
    if (d.dtype == GEMM_RS_BF16 && (d.K >= kMaxKBf16 || d.N >= kMaxNBf16))
        return GEMM_RS_ERR_UNSUPPORTED;
    int64_t tiles = ((d.M + bm - 1) / bm) * (d.N / bn);
    if (tiles * d.W > INT32_MAX) return GEMM_RS_ERR_UNSUPPORTED;
    // staging W*M*N floats must be addressable with 64-bit offsets
    if ((double)d.W * (double)d.M * (double)d.N * 4.0 > 9.0e18)
        return GEMM_RS_ERR_UNSUPPORTED;
    return GEMM_RS_OK;
}

void free_plan(gemm_rs_plan_s *p) {
    if (!p) return;
    int cur = -1;
    bool switched = false;
    if (hipGetDevice(&cur) == hipSuccess && cur != p->device)
        switched = hipSetDevice(p->device) == hipSuccess;
    // teardown is best effort: a failure here leaves nothing to undo
    (void)hipFree(p->staging);
    (void)hipFree(p->flags);
    (void)hipFree(p->counters);
    (void)hipFree(p->sub_counters);
    (void)hipFree(p->sub);
    (void)hipFree(p->sub_flags);
    (void)hipFree(p->err);
    (void)hipFree(p->trace);
    (void)hipFree(p->slot_tab);
    for (int i = 0; i < kEvents; ++i)
        if (p->slice_done[i]) (void)hipEventDestroy(p->slice_done[i]);
    if (p->aux_done) (void)hipEventDestroy(p->aux_done);
    if (p->aux) (void)hipStreamDestroy(p->aux);
    if (switched) (void)hipSetDevice(cur);
    free(p);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The plan's memory lives on one device: work is only enqueued while that
// device is current (its pointers mean nothing on another device).
bool on_plan_device(int device) {
    int cur = -1;
    return hipGetDevice(&cur) == hipSuccess && cur == device;
}

// Zero every flag, counter and the error word (plan time and after errors).
hipError_t clear_protocol_state(gemm_rs_plan_s *p, hipStream_t s) {
    hipError_t e = hipMemsetAsync(p->flags, 0, p->flags_bytes, s);
    if (e == hipSuccess) e = hipMemsetAsync(p->counters, 0, p->counters_bytes, s);
    if (e == hipSuccess && p->sub_counters)
        e = hipMemsetAsync(p->sub_counters, 0, p->counters_bytes * p->d.groups, s);
    if (e == hipSuccess && p->sub_flags)
        e = hipMemsetAsync(p->sub_flags, 0, p->sub_flags_bytes, s);
    if (e == hipSuccess) e = hipMemsetAsync(p->err, 0, 4 * sizeof(int32_t), s);
    return e;
}

// Validate a descriptor, fill in its defaults and derive the geometry and
// buffer sizes of a pass.  Host arithmetic only: no HIP call, no
// allocation (shared by the plan and the no-allocation entry point).
int resolve(const gemm_rs_desc_t &desc, gemm_rs_plan_s *p) {
    gemm_rs_desc_t d = desc;
    int32_t bm = 0, bn = 0;
    pick_default_tile(d, &bm, &bn);
    int rc = validate(d, bm, bn);
    if (rc != GEMM_RS_OK) return rc;
    d.tile_m = bm;
    d.tile_n = bn;
    // default: groups of 4 tile-rows walked column by column, so the ~32
    // tiles a rank has in flight on its XCD share 4 A and 8 B panels in L2
    if (d.group_m == 0) d.group_m = 4;
    if (d.order == GEMM_RS_ORDER_FLAT) d.groups = 1;
    if (d.timeout_ms == 0) d.timeout_ms = 1000;

    p->d = d;
    TileGeom &g = p->g;
    g.M = d.M; g.N = d.N; g.K = d.K; g.W = d.W; g.Mc = d.M / d.W;
    g.BM = bm; g.BN = bn;
    g.tiles_m = (int32_t)((d.M + bm - 1) / bm);
    g.tiles_n = (int32_t)(d.N / bn);
    g.T = g.tiles_m * g.tiles_n;
    // more tile-rows per group than the matrix has changes nothing
    g.group_m = d.group_m < g.tiles_m ? d.group_m : g.tiles_m;
    g.swizzle = d.swizzle;
    // more tiles per visit than the largest chunk holds changes nothing
    g.interleave = d.interleave > 1 ? (d.interleave < g.T ? d.interleave : g.T) : 1;
    g.bm_shift = 0;
    while ((1 << g.bm_shift) < bm) ++g.bm_shift;
    p->units_per_tile = (bm + kReduceRows - 1) / kReduceRows;

    const int staging_elem = d.staging_dtype == GEMM_RS_STAGING_BF16 ? 2 : 4;
    g.slot = staging_slot_elems(g.Mc, g.N, staging_elem);
    p->staging_bytes = (int64_t)d.W * d.W * g.slot * staging_elem;
    p->flags_bytes = (int64_t)d.W * g.T * 4;
    p->counters_bytes = (int64_t)g.T * 4;
    p->trace_bytes = (int64_t)d.W * g.T * 4;
    if (d.materialize_sub) {
        p->sub_bytes = (int64_t)d.groups * d.M * d.N * 4;
        p->sub_flags_bytes = (int64_t)d.groups * g.T * p->units_per_tile * 4;
    }
    {
        const int32_t n0 = chunk_first_tile_row(g, 1) - chunk_first_tile_row(g, 0);
        p->uniform_chunks = true;
        for (int32_t dd = 1; dd < g.W; ++dd)
            if (chunk_first_tile_row(g, dd + 1) - chunk_first_tile_row(g, dd) != n0)
                p->uniform_chunks = false;
    }
    return GEMM_RS_OK;
}

// The current device and the flag-wait bound in its wall-clock ticks.
int resolve_device(gemm_rs_plan_s *p) {
    if (hipGetDevice(&p->device) != hipSuccess) return GEMM_RS_ERR_HIP;
    int rate_khz = 0;
    if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate,
                              p->device) != hipSuccess || rate_khz <= 0)
        rate_khz = 100000;  // the 100 MHz constant clock
    p->timeout_ticks = (uint64_t)p->d.timeout_ms * (uint64_t)rate_khz;
    return GEMM_RS_OK;
}

// Enqueue one pass of plan p on stream s (checks the run flags and
// pointers, no host synchronisation, no allocation).  Without an auxiliary
// stream (p->aux == nullptr) the identity-order overlap runs serially.
int enqueue(gemm_rs_plan_s *p, const void *A, const void *B, const void *C, float alpha,
            float beta, void *out, hipStream_t s, uint32_t run_flags) {
    const uint32_t known = GEMM_RS_RUN_GEMM | GEMM_RS_RUN_REDUCE |
                           GEMM_RS_KEEP_FLAGS | GEMM_RS_TRACE_TILES |
                           GEMM_RS_OVERLAP_REDUCE | GEMM_RS_LAST_ARRIVER;
    if (run_flags & ~known) return GEMM_RS_ERR_INVALID_ARG;
    if ((run_flags & GEMM_RS_OVERLAP_REDUCE) && (run_flags & GEMM_RS_LAST_ARRIVER))
        return GEMM_RS_ERR_INVALID_ARG;
    const bool do_gemm = run_flags & GEMM_RS_RUN_GEMM;
    const bool do_reduce = run_flags & GEMM_RS_RUN_REDUCE;
    if (do_gemm) {
        // with K == 0 the operands are never read and may be NULL
        if ((p->g.K > 0 && (!A || !B)) || !aligned16(A) || !aligned16(B))
            return GEMM_RS_ERR_INVALID_ARG;
        if (p->d.has_c && (!C || !aligned16(C))) return GEMM_RS_ERR_INVALID_ARG;
        if (!p->d.has_c && C) return GEMM_RS_ERR_INVALID_ARG;
    }
    if (do_reduce && (!out || !aligned16(out))) return GEMM_RS_ERR_INVALID_ARG;

    GemmArgs a = {};   // fields this path does not use stay zero (no gate, no plain output)
    a.g = p->g;
    a.A = A; a.B = B; a.C = C;
    a.ldc = p->d.ldc;
    a.has_c = p->d.has_c;
    a.alpha = alpha; a.beta = beta;
    a.staging = p->staging;
    a.staging_bf16 = p->d.staging_dtype == GEMM_RS_STAGING_BF16;
    a.flags = p->flags;
    a.trace = (run_flags & GEMM_RS_TRACE_TILES) ? p->trace : nullptr;
    // consumers run after the producing launch completes (same stream or an
    // event dependency), so flags are published with plain stores; only the
    // last-arriver mode (a consumer in the same launch) releases them
    a.release_flags = 0;
    a.b_offset = 0;
    a.n_blocks = (uint32_t)((int64_t)p->g.W * p->g.T);
    // the W virtual ranks share one GPU: run them rank after rank across
    // the XCDs (each rank's own tile order is unchanged)
    a.xcd_rank_major = 1;
    auto gemm = [&](uint32_t b_lo, uint32_t b_hi, hipStream_t st, int coresident = 0) {
        GemmArgs x = a;
        x.b_offset = b_lo;
        x.n_blocks = b_hi - b_lo;
        x.coresident = coresident;
        // the tabulated slots hold the full launch only
        x.slot_tab = (b_lo == 0 && b_hi == a.n_blocks) ? p->slot_tab : nullptr;
        if (x.n_blocks == 0) return hipSuccess;
        return p->d.dtype == GEMM_RS_BF16 ? launch_gemm_bf16(x, st) : launch_gemm_f32(x, st);
    };

    ReduceArgs r = {};
    r.g = p->g;
    r.order = p->d.order;
    r.groups = p->d.groups;
    r.keep_flags = (run_flags & GEMM_RS_KEEP_FLAGS) ? 1 : 0;
    r.units_per_tile = p->units_per_tile;
    r.timeout_ticks = p->timeout_ticks;
    r.staging = p->staging;
    r.staging_bytes = p->staging_bytes;
    r.staging_bf16 = p->d.staging_dtype == GEMM_RS_STAGING_BF16;
    r.out = out;
    r.flags = p->flags;
    r.counters = p->counters;
    r.err = p->err;
    r.sub = p->sub;
    r.sub_flags = p->sub_flags;
    r.slice_kind = kSliceAll;
    r.k_lo = r.k_hi = 0;

    const bool overlap_req = (run_flags & GEMM_RS_OVERLAP_REDUCE) && do_gemm && do_reduce &&
                             !p->d.materialize_sub && p->uniform_chunks;
    // remote-first order: owner-fused reduce in the last step
    const bool fused = overlap_req && p->d.swizzle == GEMM_RS_SWIZZLE_REMOTE_FIRST &&
                       p->d.dtype == GEMM_RS_BF16 && !(run_flags & GEMM_RS_KEEP_FLAGS) &&
                       fused_reduce_supported(p->g.BM, p->g.BN, p->g.W);
    // identity order: chunk-by-chunk slices reduced on the second stream
    const bool sliced = overlap_req && p->d.swizzle == GEMM_RS_SWIZZLE_IDENTITY && p->aux;
    // one launch: each tile's last producer sums it
    const bool last_arriver = (run_flags & GEMM_RS_LAST_ARRIVER) && do_gemm && do_reduce &&
                              !p->d.materialize_sub && p->d.dtype == GEMM_RS_BF16 &&
                              fused_reduce_supported(p->g.BM, p->g.BN, p->g.W);
    hipError_t e = hipSuccess;
    if (last_arriver) {
        GemmArgs x = a;
        x.slot_tab = p->slot_tab;   // the full launch
        x.fuse_reduce = kFuseLastArriver;
        x.release_flags = 1;
        // fp32 staging below 4 GiB: written through past L2 by buffer
        // stores, so the producers' release has no dirty lines to flush
        x.stage_wt = (p->staging_bytes <= (int64_t)0xffffffffu &&
                      p->d.staging_dtype == GEMM_RS_STAGING_F32) ? 1 : 0;
        x.staging_bytes = p->staging_bytes;
        x.counters = p->counters;
        x.keep_flags = (run_flags & GEMM_RS_KEEP_FLAGS) ? 1 : 0;
        x.groups = p->d.groups;
        x.out = out;
        x.err = p->err;
        e = launch_gemm_bf16(x, s);
        return e == hipSuccess ? GEMM_RS_OK : GEMM_RS_ERR_HIP;
    }
    if (fused) {
        // Every rank visits its own chunk last, so rank d's last n = T/W
        // tiles (the tiles of chunk d) are the last contribution to each of
        // those tiles, and every other rank's partial of them comes from an
        // earlier step.  The earlier steps run as one launch; the last step
        // runs as a second launch on the same stream whose workgroups each
        // sum their tile's partials and write the output directly (no
        // separate reduce, and the own partial is never staged).
        const uint32_t W = (uint32_t)p->g.W, T = (uint32_t)p->g.T;
        const uint32_t k0 = T - T / W;
        e = gemm(0, W * k0, s);
        if (e == hipSuccess) {
            GemmArgs x = a;
            x.b_offset = W * k0;
            x.n_blocks = W * (T - k0);
            x.fuse_reduce = kFuseOwner;
            x.groups = p->d.groups;
            x.out = out;
            x.err = p->err;
            x.timeout_ticks = p->timeout_ticks;
            e = launch_gemm_bf16(x, s);
        }
        return e == hipSuccess ? GEMM_RS_OK : GEMM_RS_ERR_HIP;
    }
    if (sliced) {
        const uint32_t W = (uint32_t)p->g.W, T = (uint32_t)p->g.T;
        const uint32_t n = T / W;   // tiles per chunk (uniform)
        // GEMM steps [q0, q1) of every rank, then the reduce of the tiles
        // they completed on the auxiliary stream, concurrent with the next
        // GEMM slice.  Every rank computes chunk c in steps [c*n, (c+1)*n),
        // so chunk c is complete after them; chunks are grouped into at
        // most kChunkSlices slices.
        const uint32_t parts = W < (uint32_t)kChunkSlices ? W : (uint32_t)kChunkSlices;
        for (uint32_t j = 0; j < parts && e == hipSuccess; ++j) {
            const uint32_t q0 = n * ((W * j) / parts), q1 = n * ((W * (j + 1)) / parts);
            e = gemm(W * q0, W * q1, s, 1);
            if (e == hipSuccess) e = hipEventRecord(p->slice_done[j], s);
            if (e == hipSuccess) e = hipStreamWaitEvent(p->aux, p->slice_done[j], 0);
            if (e == hipSuccess) {
                ReduceArgs rs = r;
                rs.slice_kind = kSliceSteps;
                rs.k_lo = q0;
                rs.k_hi = q1;
                e = launch_reduce(rs, p->d.dtype, p->aux);
            }
        }
        if (e == hipSuccess) e = hipEventRecord(p->aux_done, p->aux);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, p->aux_done, 0);
        return e == hipSuccess ? GEMM_RS_OK : GEMM_RS_ERR_HIP;
    }

    if (do_gemm) e = gemm(0, a.n_blocks, s);
    if (e == hipSuccess && do_reduce) {
        if (p->d.materialize_sub) {
            ReduceArgs rs = r;
            rs.counters = p->sub_counters;
            e = launch_reduce_sub(rs, s);
            if (e == hipSuccess) e = launch_reduce_final_sub(r, p->d.dtype, s);
        } else {
            e = launch_reduce(r, p->d.dtype, s);
        }
    }
    return e == hipSuccess ? GEMM_RS_OK : GEMM_RS_ERR_HIP;
}


// ---- workspace of the no-allocation entry point ----
// One static device array: every GPU the library runs on holds its own copy
// until the process ends, and every gemm_rs_run_noalloc call on that GPU
// shares it.  In host code the array's name is not a device address; the
// address comes from hipGetSymbolAddress, once per device, and only that
// pointer is handed to kernels.
constexpr int kMaxScratchDevices = 64;
std::once_flag scratch_once[kMaxScratchDevices];
void *scratch_ptr[kMaxScratchDevices];
hipError_t scratch_rc[kMaxScratchDevices];

// The current device's copy of the scratch array (looked up on the first
// call made with that device current).
hipError_t device_scratch(int dev, unsigned char **ptr) {
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::call_once(scratch_once[dev], [dev] {
        void *q = nullptr;
        const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        scratch_rc[dev] = e;
        scratch_ptr[dev] = e == hipSuccess ? q : nullptr;
    });
    *ptr = (unsigned char *)scratch_ptr[dev];
    return scratch_rc[dev];
}

int64_t align256(int64_t n) { return (n + 255) & ~int64_t(255); }

}  // namespace

extern "C" {

const char *gemm_rs_strerror(int code) {
    switch (code) {
    case GEMM_RS_OK: return "ok";
    case GEMM_RS_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_RS_ERR_UNSUPPORTED: return "unsupported configuration";
    case GEMM_RS_ERR_HIP: return "HIP runtime error";
    case GEMM_RS_ERR_TIMEOUT: return "device flag wait timed out";
    case GEMM_RS_ERR_PROTOCOL: return "flag protocol violation";
    case GEMM_RS_ERR_SCRATCH:
        return "workspace larger than the static scratch of gemm_rs_run_noalloc";
    default: return "unknown status";
    }
}

int gemm_rs_plan(const gemm_rs_desc_t *desc, gemm_rs_plan_t *out) {
    if (out) *out = nullptr;
    if (!desc || !out) return GEMM_RS_ERR_INVALID_ARG;
    gemm_rs_plan_s *p = (gemm_rs_plan_s *)calloc(1, sizeof(gemm_rs_plan_s));
    if (!p) return GEMM_RS_ERR_HIP;
    int rc = resolve(*desc, p);
    if (rc == GEMM_RS_OK) rc = resolve_device(p);
    if (rc != GEMM_RS_OK) {
        free(p);
        return rc;
    }
    const gemm_rs_desc_t &d = p->d;
    hipError_t e = hipMalloc(&p->staging, p->staging_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->flags, p->flags_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->counters, p->counters_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->err, 4 * sizeof(int32_t));
    if (e == hipSuccess) e = hipMalloc(&p->trace, p->trace_bytes);
    // the slot table packs the tile id in 26 bits; larger grids derive it
    if (e == hipSuccess && p->g.T < (1 << kSlotTileBits))
        e = hipMalloc(&p->slot_tab, p->trace_bytes);
    if (e == hipSuccess && d.materialize_sub) {
        e = hipMalloc(&p->sub, p->sub_bytes);
        if (e == hipSuccess) e = hipMalloc(&p->sub_flags, p->sub_flags_bytes);
        if (e == hipSuccess)
            e = hipMalloc(&p->sub_counters, p->counters_bytes * d.groups);
    }
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->aux, hipStreamNonBlocking);
    for (int i = 0; i < kEvents && e == hipSuccess; ++i)
        e = hipEventCreateWithFlags(&p->slice_done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->aux_done, hipEventDisableTiming);
    // flags are zeroed once, here; runs keep them at 0 between passes.  The
    // zeroing runs on the plan's own stream and only that stream is waited
    // for (unrelated work on the device is not)
    if (e == hipSuccess) e = clear_protocol_state(p, p->aux);
    if (e == hipSuccess) e = hipMemsetAsync(p->trace, 0xff, p->trace_bytes, p->aux);
    if (e == hipSuccess && p->slot_tab) e = launch_slot_table(p->g, p->slot_tab, p->aux);
    if (e == hipSuccess) e = hipStreamSynchronize(p->aux);
    if (e != hipSuccess) {
        free_plan(p);
        return GEMM_RS_ERR_HIP;
    }
    *out = p;
    return GEMM_RS_OK;
}

int gemm_rs_destroy(gemm_rs_plan_t p) {
    free_plan(p);
    return GEMM_RS_OK;
}

int gemm_rs_query(gemm_rs_plan_t p, gemm_rs_info_t *info) {
    if (!p || !info) return GEMM_RS_ERR_INVALID_ARG;
    memset(info, 0, sizeof(*info));
    info->Mc = p->g.Mc;
    info->tile_m = p->g.BM;
    info->tile_n = p->g.BN;
    info->tiles_m = p->g.tiles_m;
    info->tiles_n = p->g.tiles_n;
    info->T = p->g.T;
    info->group_m = p->g.group_m;
    info->staging = p->staging;
    info->flags = p->flags;
    info->sub = p->sub;
    info->sub_flags = p->sub_flags;
    info->trace = p->trace;
    info->staging_bytes = p->staging_bytes;
    info->flags_bytes = p->flags_bytes;
    info->sub_bytes = p->sub_bytes;
    info->sub_flags_bytes = p->sub_flags_bytes;
    info->slot_elems = p->g.slot;
    info->workspace_bytes = p->staging_bytes + p->flags_bytes +
                            p->counters_bytes * (1 + (p->sub_counters ? p->d.groups : 0)) +
                            p->sub_bytes + p->sub_flags_bytes + p->trace_bytes + 16;
    return GEMM_RS_OK;
}

int gemm_rs_run(gemm_rs_plan_t p, const void *A, const void *B, const void *C,
                float alpha, float beta, void *out, void *stream,
                uint32_t run_flags) {
    if (!p || !on_plan_device(p->device)) return GEMM_RS_ERR_INVALID_ARG;
    return enqueue(p, A, B, C, alpha, beta, out, (hipStream_t)stream, run_flags);
}

int gemm_rs_run_noalloc(const gemm_rs_desc_t *desc, const void *A, const void *B,
                        const void *C, float alpha, float beta, void *out, void *stream,
                        uint32_t run_flags, int32_t *status) {
    if (!desc) return GEMM_RS_ERR_INVALID_ARG;
    const uint32_t allowed = GEMM_RS_RUN_ALL | GEMM_RS_OVERLAP_REDUCE | GEMM_RS_LAST_ARRIVER;
    if ((run_flags & GEMM_RS_RUN_ALL) != GEMM_RS_RUN_ALL || (run_flags & ~allowed))
        return GEMM_RS_ERR_INVALID_ARG;
    if (status && ((uintptr_t)status & 15u)) return GEMM_RS_ERR_INVALID_ARG;
    gemm_rs_plan_s p;
    memset(&p, 0, sizeof p);
    int rc = resolve(*desc, &p);
    if (rc != GEMM_RS_OK) return rc;
    if (p.d.materialize_sub) return GEMM_RS_ERR_UNSUPPORTED;
    // layout: error record | flags [W][T] | counters [T] | staging
    const int64_t off_flags = 256;
    const int64_t off_counters = off_flags + align256(p.flags_bytes);
    const int64_t off_staging = off_counters + align256(p.counters_bytes);
    if (off_staging + p.staging_bytes > (int64_t)kScratchBytes) return GEMM_RS_ERR_SCRATCH;
    rc = resolve_device(&p);
    if (rc != GEMM_RS_OK) return rc;
    unsigned char *base = nullptr;
    if (device_scratch(p.device, &base) != hipSuccess || !base) return GEMM_RS_ERR_HIP;
    p.err = status ? status : (int32_t *)base;
    p.flags = (uint32_t *)(base + off_flags);
    p.counters = (uint32_t *)(base + off_counters);
    p.staging = base + off_staging;
    hipStream_t s = (hipStream_t)stream;
    // the array keeps the previous call's contents: flags, counters and
    // the error record start every call at zero (flags and counters are
    // one contiguous range)
    const hipError_t e =
        launch_clear_words(p.flags, (off_staging - off_flags) / 4, (uint32_t *)p.err, 4, s);
    if (e != hipSuccess) return GEMM_RS_ERR_HIP;
    return enqueue(&p, A, B, C, alpha, beta, out, s, run_flags);
}

int gemm_rs_tile_order(gemm_rs_plan_t p, int32_t *host_trace) {
    if (!p || !host_trace || !on_plan_device(p->device)) return GEMM_RS_ERR_INVALID_ARG;
    hipError_t e = launch_tile_order(p->g, p->trace, nullptr);
    if (e == hipSuccess)
        e = hipMemcpy(host_trace, p->trace, p->trace_bytes, hipMemcpyDeviceToHost);
    return e == hipSuccess ? GEMM_RS_OK : GEMM_RS_ERR_HIP;
}

int gemm_rs_status(gemm_rs_plan_t p, void *stream, int32_t *detail) {
    if (!p || !on_plan_device(p->device)) return GEMM_RS_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    int32_t e4[4] = {0, 0, 0, 0};
    if (hipStreamSynchronize(s) != hipSuccess) return GEMM_RS_ERR_HIP;
    if (hipMemcpy(e4, p->err, sizeof e4, hipMemcpyDeviceToHost) != hipSuccess)
        return GEMM_RS_ERR_HIP;
    if (detail) memcpy(detail, e4, sizeof e4);
    if (e4[0] != 0) {
        if (clear_protocol_state(p, s) != hipSuccess) return GEMM_RS_ERR_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return GEMM_RS_ERR_HIP;
    }
    return e4[0];
}

}  // extern "C"
