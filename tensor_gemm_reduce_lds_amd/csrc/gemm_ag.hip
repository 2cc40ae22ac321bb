// All-gather fused into the GEMM prologue (include/gemm_ag.h).
//
// The gather is issued tile-row by tile-row in each rank's send order and
// every finished tile-row publishes a 32-bit signal; each GEMM workgroup
// waits for the signal of the tile-row of X it multiplies before its
// mainloop (page "flux精读", section 3 Design: the all-gather runs as
// copies with a signal per tile, and thread blocks wait on their tile's
// signal in the order the tiles are sent; section 4.2: 32-bit signals
// allocated once).  On one GPU the copies are a kernel on a second stream
// standing in for the DMA transfers.
#include <stdlib.h>

#include "gemm_ag.h"
#include "gemm_rs_internal.h"

using namespace gemm_rs;

namespace {

constexpr int kCopyThreads = 256;
// each tile-row of X is copied as kSubBlocks pieces (a power of two, so the
// per-tile-row arrival counters stay consistent across 32-bit wrap-around)
constexpr uint32_t kSubBlocks = 16;
static_assert((kSubBlocks & (kSubBlocks - 1)) == 0, "power of two");
// The copy grid is enqueued before the gated GEMM, so its progress does not
// rest on finding room beside waiting GEMM tiles; its waves still fit in the
// registers every GEMM tile configuration leaves free on a SIMD at its own
// maximum occupancy (the test suite checks this against the compiler's
// resource report), so copies keep running while GEMM tiles hold the CUs.
// Workgroups of the persistent copy grid: one per CU.
constexpr uint32_t kCopyGrid = 256;

struct AgCopyArgs {
    TileGeom g;
    const uint16_t *X;    // [M][K] (the W row shards stacked)
    uint16_t *gathered;   // [W][M][K]
    uint32_t *signals;    // [W][tiles_m]
    uint32_t *arrived;    // [W][tiles_m] sub-blocks copied, over all runs
    uint32_t epoch;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Tile-row sent k-th to rank r: its own chunk's tile-rows first, then those
// of chunks r+1, r+2, ... (mod W), each chunk's tile-rows in ascending order
// (a tile-row belongs to the chunk of its first row).
__device__ int32_t send_order_tile_row(const TileGeom &g, int32_t r, uint32_t k) {
    for (int32_t s = 0; s < g.W; ++s) {
        const int32_t c = (r + s) % g.W;
        const int32_t lo = chunk_first_tile_row(g, c);
        const uint32_t n = (uint32_t)(chunk_first_tile_row(g, c + 1) - lo);
        if (k < n) return lo + (int32_t)k;
        k -= n;
    }
    return 0;   // unreachable for k < tiles_m
}

// A persistent grid walks the copy items in send order: item
// i = (k*W + r)*kSubBlocks + sub is sub-block `sub` of the tile-row sent
// k-th to rank r, so every rank's first tile-rows arrive first.  The
// workgroup that completes a tile-row's last sub-block publishes
// signal[r][tm] = epoch: each piece ends with an agent-scope release add on
// the tile-row's arrival counter, and the add that completes the count is
// followed by an acquire fence and the release store of the signal, so a
// reader that acquires the signal sees every piece's rows.
__global__ __launch_bounds__(kCopyThreads) void ag_copy_kernel(AgCopyArgs a) {
    const TileGeom &g = a.g;
    const uint32_t items = (uint32_t)g.W * (uint32_t)g.tiles_m * kSubBlocks;
    for (uint32_t i = blockIdx.x; i < items; i += gridDim.x) {
        const uint32_t sub = i % kSubBlocks;
        const uint32_t piece = i / kSubBlocks;
        const int32_t r = (int32_t)(piece % (uint32_t)g.W);
        const int32_t tm = send_order_tile_row(g, r, piece / (uint32_t)g.W);
        const int64_t row_lo = (int64_t)tm * g.BM;
        const int64_t row_hi = row_lo + g.BM < g.M ? row_lo + g.BM : g.M;
        // rows [row_lo, row_hi) of X are one contiguous run of 16-byte
        // words; this item copies the sub-th of kSubBlocks equal parts
        const int64_t n16 = (row_hi - row_lo) * g.K / 8;
        const int64_t lo16 = n16 * sub / kSubBlocks, hi16 = n16 * (sub + 1) / kSubBlocks;
        const u32x4_t *src = (const u32x4_t *)(a.X + row_lo * g.K);
        u32x4_t *dst = (u32x4_t *)(a.gathered + ((int64_t)r * g.M + row_lo) * g.K);
        // software-pipelined in stages of 2 words per thread: the next
        // stage's loads are issued before the current stage's stores, so
        // the loads never wait behind stores (one in-order memory counter)
        constexpr int64_t kStage = 2 * kCopyThreads;
        const int64_t full_end = lo16 + (hi16 - lo16) / kStage * kStage;
        int64_t j = lo16 + threadIdx.x;
        if (lo16 + kStage <= full_end) {
            u32x4_t c0 = src[j], c1 = src[j + kCopyThreads];
            for (j += kStage; j < full_end; j += kStage) {
                const u32x4_t n0 = src[j], n1 = src[j + kCopyThreads];
                dst[j - kStage] = c0;
                dst[j - kStage + kCopyThreads] = c1;
                c0 = n0;
                c1 = n1;
            }
            dst[j - kStage] = c0;
            dst[j - kStage + kCopyThreads] = c1;
        }
        for (; j < hi16; j += kCopyThreads) dst[j] = src[j];
        // every wave's stores of this item have completed before the barrier
        __syncthreads();
        if (threadIdx.x == 0) {
            const int64_t f = (int64_t)r * g.tiles_m + tm;
            const uint32_t before = __hip_atomic_fetch_add(&a.arrived[f], 1u, __ATOMIC_RELEASE,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            if ((before + 1u) % kSubBlocks == 0) {
                // the last piece: acquire the other pieces' releases (this
                // add read their release sequence), then publish the tile-row
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                __hip_atomic_store(&a.signals[f], a.epoch, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

hipError_t launch_ag_copy(const AgCopyArgs &a, hipStream_t s) {
    const uint32_t items = (uint32_t)a.g.W * (uint32_t)a.g.tiles_m * kSubBlocks;
    const uint32_t grid = items < kCopyGrid ? items : kCopyGrid;
    hipLaunchKernelGGL(ag_copy_kernel, dim3(grid), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

struct gemm_ag_plan_s {
    gemm_ag_desc_t d;       // resolved (tile, group_m, timeout filled in)
    TileGeom g;
    int device;
    uint64_t timeout_ticks;
    uint16_t *gathered;     // [W][M][K]
    uint32_t *signals;      // [W][tiles_m]
    uint32_t *arrived;      // [W][tiles_m] sub-blocks copied (counts up across runs)
    int32_t *err;           // {code, rank, tile-row, 0}
    int64_t gathered_bytes, signals_bytes;
    uint32_t epoch;         // value the latest copy published
    hipStream_t copy;       // the second stream (default priority)
    hipEvent_t ready, copied;
};

namespace {

constexpr int64_t kKStepAg = 64;

void free_ag(gemm_ag_plan_s *p) {
    if (!p) return;
    int cur = -1;
    bool switched = false;
    if (hipGetDevice(&cur) == hipSuccess && cur != p->device)
        switched = hipSetDevice(p->device) == hipSuccess;
    // teardown is best effort: a failure here leaves nothing to undo
    (void)hipFree(p->gathered);
    (void)hipFree(p->signals);
    (void)hipFree(p->arrived);
    (void)hipFree(p->err);
    if (p->ready) (void)hipEventDestroy(p->ready);
    if (p->copied) (void)hipEventDestroy(p->copied);
    if (p->copy) (void)hipStreamDestroy(p->copy);
    if (switched) (void)hipSetDevice(cur);
    free(p);
}

int validate_ag(const gemm_ag_desc_t &d, int32_t bm, int32_t bn) {
    if (d.W < 1 || d.W > 64 || d.M < 1 || d.N < 1 || d.K < 1) return GEMM_RS_ERR_INVALID_ARG;
    if (d.M % d.W != 0) return GEMM_RS_ERR_INVALID_ARG;
    if (d.group_m < 0 || d.tile_m < 0 || d.tile_n < 0 || d.pad != 0)
        return GEMM_RS_ERR_INVALID_ARG;
    if (!bf16_tile_supported(bm, bn)) return GEMM_RS_ERR_UNSUPPORTED;
    if (d.N % bn != 0 || d.K % kKStepAg != 0) return GEMM_RS_ERR_UNSUPPORTED;
    if (d.M > INT32_MAX || d.N > INT32_MAX || d.K > INT32_MAX) return GEMM_RS_ERR_UNSUPPORTED;
    // 32-bit buffer offsets of the GEMM's per-step operand windows
    if (d.K >= (int64_t(1) << 23) || d.N >= (int64_t(1) << 25)) return GEMM_RS_ERR_UNSUPPORTED;
    const int64_t tiles_m = (d.M + bm - 1) / bm;
    if (tiles_m * (d.N / bn) * d.W > INT32_MAX) return GEMM_RS_ERR_UNSUPPORTED;
    // copy items are counted in 32 bits
    if (tiles_m * d.W * (int64_t)kSubBlocks > (int64_t)UINT32_MAX) return GEMM_RS_ERR_UNSUPPORTED;
    if ((double)d.W * (double)d.M * (double)d.K * 2.0 > 9.0e18) return GEMM_RS_ERR_UNSUPPORTED;
    return GEMM_RS_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// work is only enqueued while the plan's device is current
bool on_plan_device(int device) {
    int cur = -1;
    return hipGetDevice(&cur) == hipSuccess && cur == device;
}

}  // namespace

extern "C" {

int gemm_ag_plan(const gemm_ag_desc_t *desc, gemm_ag_plan_t *out) {
    if (!desc || !out) return GEMM_RS_ERR_INVALID_ARG;
    *out = nullptr;
    gemm_ag_desc_t d = *desc;
    int32_t bm = d.tile_m, bn = d.tile_n;
    if (bm == 0) bm = d.M <= 64 ? 64 : 256;
    if (bn == 0) bn = bm == 64 ? 128 : (d.N % 256 == 0 ? 256 : 128);
    const int rc = validate_ag(d, bm, bn);
    if (rc != GEMM_RS_OK) return rc;
    d.tile_m = bm;
    d.tile_n = bn;
    if (d.group_m == 0) d.group_m = 4;
    if (d.timeout_ms == 0) d.timeout_ms = 1000;

    gemm_ag_plan_s *p = (gemm_ag_plan_s *)calloc(1, sizeof(gemm_ag_plan_s));
    if (!p) return GEMM_RS_ERR_HIP;
    p->d = d;
    TileGeom &g = p->g;
    g.M = d.M; g.N = d.N; g.K = d.K; g.W = d.W; g.Mc = d.M / d.W;
    g.BM = bm; g.BN = bn;
    g.tiles_m = (int32_t)((d.M + bm - 1) / bm);
    g.tiles_n = (int32_t)(d.N / bn);
    g.T = g.tiles_m * g.tiles_n;
    g.group_m = d.group_m < g.tiles_m ? d.group_m : g.tiles_m;
    // each rank first multiplies its own chunk of X, then the chunks in the
    // order they are sent to it
    g.swizzle = GEMM_RS_SWIZZLE_SELF_FIRST;
    g.interleave = 1;
    g.bm_shift = 0;
    while ((1 << g.bm_shift) < bm) ++g.bm_shift;

    if (hipGetDevice(&p->device) != hipSuccess) { free(p); return GEMM_RS_ERR_HIP; }
    int rate_khz = 0;
    if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, p->device) !=
            hipSuccess || rate_khz <= 0)
        rate_khz = 100000;
    p->timeout_ticks = (uint64_t)d.timeout_ms * (uint64_t)rate_khz;

    p->gathered_bytes = (int64_t)d.W * d.M * d.K * 2;
    p->signals_bytes = (int64_t)d.W * g.tiles_m * 4;
    hipError_t e = hipMalloc(&p->gathered, p->gathered_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->signals, p->signals_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->arrived, p->signals_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->err, 16);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->copy, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->copied, hipEventDisableTiming);
    // signals are zeroed once; every later run publishes a new epoch.  The
    // zeroing runs on the plan's own stream and only that stream is waited
    // for (unrelated work on the device is not)
    if (e == hipSuccess) e = hipMemsetAsync(p->signals, 0, p->signals_bytes, p->copy);
    if (e == hipSuccess) e = hipMemsetAsync(p->arrived, 0, p->signals_bytes, p->copy);
    if (e == hipSuccess) e = hipMemsetAsync(p->err, 0, 16, p->copy);
    if (e == hipSuccess) e = hipStreamSynchronize(p->copy);
    if (e != hipSuccess) {
        free_ag(p);
        return GEMM_RS_ERR_HIP;
    }
    *out = p;
    return GEMM_RS_OK;
}

int gemm_ag_run(gemm_ag_plan_t p, const void *X, const void *B, void *out, void *stream,
                uint32_t run_flags) {
    if (!p || !on_plan_device(p->device)) return GEMM_RS_ERR_INVALID_ARG;
    const uint32_t known = GEMM_AG_RUN_COPY | GEMM_AG_RUN_GEMM | GEMM_AG_FUSED |
                           GEMM_AG_EXPECT_NEXT;
    if (run_flags & ~known) return GEMM_RS_ERR_INVALID_ARG;
    const bool do_copy = run_flags & GEMM_AG_RUN_COPY;
    const bool do_gemm = run_flags & GEMM_AG_RUN_GEMM;
    if (do_copy && (!X || !aligned16(X))) return GEMM_RS_ERR_INVALID_ARG;
    if (do_gemm && (!B || !out || !aligned16(B) || !aligned16(out)))
        return GEMM_RS_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;

    uint32_t wait_epoch = p->epoch;
    if (do_copy) {
        p->epoch = p->epoch + 1 == 0 ? 1 : p->epoch + 1;   // 0 is the initial state
        wait_epoch = p->epoch;
    } else if (run_flags & GEMM_AG_EXPECT_NEXT) {
        wait_epoch = p->epoch + 1 == 0 ? 1 : p->epoch + 1;
    }

    AgCopyArgs c = {};
    c.g = p->g;
    c.X = (const uint16_t *)X;
    c.gathered = p->gathered;
    c.signals = p->signals;
    c.arrived = p->arrived;
    c.epoch = p->epoch;

    GemmArgs a = {};
    a.g = p->g;
    a.A = p->gathered;
    a.B = B;
    a.C = nullptr;
    a.ldc = 0;
    a.has_c = 0;
    a.alpha = 1.0f;
    a.beta = 0.0f;
    a.staging = out;
    a.staging_bf16 = 1;
    a.flags = nullptr;
    a.trace = nullptr;
    a.release_flags = 0;
    a.b_offset = 0;
    a.n_blocks = (uint32_t)(p->g.W * p->g.T);
    a.plain_out = 1;
    // fused: tiles run rank-interleaved, the order the copies deliver
    // tile-rows in; otherwise every tile-row is already there and the
    // XCD map of the reduce-scatter GEMM applies
    a.xcd_rank_major = (do_copy && (run_flags & GEMM_AG_FUSED)) ? 0 : 1;
    a.signals = p->signals;
    a.epoch = wait_epoch;
    a.timeout_ticks = p->timeout_ticks;
    a.err = p->err;

    hipError_t e = hipSuccess;
    if (do_copy && do_gemm && (run_flags & GEMM_AG_FUSED)) {
        // the copies start once earlier work on `stream` (which wrote X) is
        // done, on the second stream, while the GEMM's tiles wait for them.
        // The copy kernel is enqueued first: it waits for nothing, so its
        // workgroups take their places before the gated GEMM's fill the
        // CUs, and progress does not rest on the copies finding room beside
        // waiting GEMM workgroups (which the register budget also leaves).
        e = hipEventRecord(p->ready, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(p->copy, p->ready, 0);
        if (e == hipSuccess) e = launch_ag_copy(c, p->copy);
        if (e == hipSuccess) e = launch_gemm_bf16(a, s);
        if (e == hipSuccess) e = hipEventRecord(p->copied, p->copy);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, p->copied, 0);
    } else {
        if (do_copy) e = launch_ag_copy(c, s);
        if (e == hipSuccess && do_gemm) e = launch_gemm_bf16(a, s);
    }
    return e == hipSuccess ? GEMM_RS_OK : GEMM_RS_ERR_HIP;
}

int gemm_ag_query(gemm_ag_plan_t p, gemm_ag_info_t *info) {
    if (!p || !info) return GEMM_RS_ERR_INVALID_ARG;
    info->tile_m = p->g.BM;
    info->tile_n = p->g.BN;
    info->tiles_m = p->g.tiles_m;
    info->tiles_n = p->g.tiles_n;
    info->group_m = p->g.group_m;
    info->epoch = p->epoch;
    info->gathered = p->gathered;
    info->signals = p->signals;
    info->gathered_bytes = p->gathered_bytes;
    return GEMM_RS_OK;
}

int gemm_ag_status(gemm_ag_plan_t p, void *stream, int32_t *detail) {
    if (!p || !on_plan_device(p->device)) return GEMM_RS_ERR_INVALID_ARG;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize(p->copy);
    int32_t h[4] = {0, 0, 0, 0};
    if (e == hipSuccess) e = hipMemcpy(h, p->err, 16, hipMemcpyDeviceToHost);
    if (e == hipSuccess && h[0] != 0) e = hipMemset(p->err, 0, 16);
    if (e != hipSuccess) return GEMM_RS_ERR_HIP;
    if (detail)
        for (int i = 0; i < 4; ++i) detail[i] = h[i];
    return h[0];
}

int gemm_ag_destroy(gemm_ag_plan_t p) {
    free_ag(p);
    return GEMM_RS_OK;
}

}  // extern "C"
