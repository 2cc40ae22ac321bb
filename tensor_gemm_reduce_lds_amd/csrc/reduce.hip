// Flag-gated, fixed-order W-way reduction of the staging slots.
//
// Work unit: up to kReduceRows rows of one tile.  A unit first waits until
// every rank's flag for its tile reads 1 (bounded by a timeout on the
// constant-rate device clock; the producers ran in an earlier launch on the
// stream), then sums the W fp32 slots of
// each element in a fixed order and writes the rank's chunk rows of `out`.
// The last unit of a tile to pass the wait puts the tile's flags back to 0,
// so no buffer is ever cleared between runs (page "flux实现：sm80 gemm+rs",
// section "cutlass自定义epilogue–sm80": the consumer waits on the
// producer's per-tile flag; section "自己的类flux实现": the pre-clear of
// the reduce buffer and the syncs around it are the cost being removed).
//
// Orders: flat y = ((S_0 + S_1) + ...) + S_{W-1}; two-level with G groups
// of L = W/G contiguous ranks: each group summed in ascending rank, then
// the group sums in ascending group (page "flux实现：sm80 gemm+rs", section
// "2D Ring优化": partial sums inside a level first, then across levels).
#include "gemm_rs_internal.h"

namespace gemm_rs {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Threads [0, count) each wait on one flag; true if all ready.  The
// producers finished in an earlier launch on the stream, whose boundary
// already makes their stores visible, so relaxed loads suffice.
__device__ bool wait_flags(uint32_t *base, int64_t stride, int count,
                           uint64_t timeout_ticks, int32_t *err, int32_t rank0,
                           int32_t tile) {
    int failed = 0;
    const int i = threadIdx.x;
    if (i < count)
        failed = wait_flag_set(base + (int64_t)i * stride, timeout_ticks, err, rank0 + i, tile);
    return !__syncthreads_or(failed);
}

__device__ __forceinline__ void store_out4(void *out, int64_t idx, f32x4_t y, bool bf16) {
    if (bf16) {
        // fptrunc to bfloat16 rounds to nearest even (v_cvt_pk_bf16_f32)
        __bf16 h0 = (__bf16)y[0], h1 = (__bf16)y[1], h2 = (__bf16)y[2], h3 = (__bf16)y[3];
        uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
        // a relaxed agent-scope store is written through past this XCD's
        // L2 (sc1): measured ~2.5% faster than a write-back store for this
        // read-mostly stream, where every write interleaved with the reads
        // costs HBM read/write turnarounds
        __hip_atomic_store((uint64_t *)((uint16_t *)out + idx),
                           (uint64_t)w0 | ((uint64_t)w1 << 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *(f32x4_t *)((float *)out + idx) = y;
    }
}

// Row range of unit `slab` of tile-row tm.
__device__ __forceinline__ void unit_rows(const TileGeom &g, int32_t tm, int32_t slab,
                                          int64_t *lo, int64_t *hi) {
    const int64_t tile_lo = (int64_t)tm * g.BM;
    int64_t tile_hi = tile_lo + g.BM;
    if (tile_hi > g.M) tile_hi = g.M;
    *lo = tile_lo + (int64_t)slab * kReduceRows;
    *hi = *lo + kReduceRows < tile_hi ? *lo + kReduceRows : tile_hi;
}

// Where the slots are read from.  Each loader returns the four consecutive
// staged elements at element index `idx` as floats.
//   PtrSlots<false>: a 16-byte non-temporal load of floats.
//   PtrSlots<true>:  an 8-byte load of four bfloat16 values, widened exactly
//                    (a bfloat16 is the top half of a float).
//   BufSlots:        a 16-byte non-temporal buffer load through one
//                    descriptor over the whole staging, with a 32-bit byte
//                    offset per lane (staging below 4 GiB).  Measured ~1%
//                    faster than the pointer form inside GEMM -> reduce
//                    steps (less 64-bit address arithmetic per load), and a
//                    load past the staging's end returns zeros.
template <bool SB>
struct PtrSlots {
    const void *S;
    __device__ __forceinline__ f32x4_t operator()(int64_t idx) const {
        if constexpr (SB) {
            const u32x2_t h =
                __builtin_nontemporal_load((const u32x2_t *)((const uint16_t *)S + idx));
            f32x4_t v;
            v[0] = __uint_as_float(h[0] << 16);
            v[1] = __uint_as_float(h[0] & 0xffff0000u);
            v[2] = __uint_as_float(h[1] << 16);
            v[3] = __uint_as_float(h[1] & 0xffff0000u);
            return v;
        } else {
            return __builtin_nontemporal_load((const f32x4_t *)((const float *)S + idx));
        }
    }
};

constexpr int kCachePolicyNT = 2;   // the nt bit of a buffer access's cache policy

struct BufSlots {
    __amdgpu_buffer_rsrc_t rs;
    __device__ __forceinline__ BufSlots(const void *S, int64_t bytes)
        : rs(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(S), (short)0,
                                               (int)(uint32_t)bytes, 0x00020000)) {}
    __device__ __forceinline__ f32x4_t operator()(int64_t idx) const {
        return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, (int)(uint32_t)(idx * 4), 0, kCachePolicyNT));
    }
};

// Sum of one element group (4 columns) over the W slots in the fixed order.
// Slot q of the element group starts at element idx + q*stride.  WT > 0:
// W == WT, unrolled; LT > 0: the group length L == LT, so the group
// boundaries fold at compile time (LT == 0: L at run time).
template <int WT, int LT, class LD>
__device__ __forceinline__ f32x4_t ordered_sum(const LD &ld, int64_t idx, int64_t stride,
                                               int W, int L_rt) {
    const int L = LT > 0 ? LT : L_rt;
    if constexpr (WT > 0) {
        f32x4_t v[WT];
#pragma unroll
        for (int q = 0; q < WT; ++q) v[q] = ld(idx + q * stride);
        f32x4_t y = v[0], s = v[0];
#pragma unroll
        for (int q = 0; q < WT; ++q) {
            s = (q % L == 0) ? v[q] : s + v[q];
            if (q % L == L - 1) y = (q / L == 0) ? s : y + s;
        }
        return y;
    } else {
        f32x4_t y = {0, 0, 0, 0}, s = {0, 0, 0, 0};
        for (int q = 0; q < W; ++q) {
            const f32x4_t v = ld(idx + q * stride);
            s = (q % L == 0) ? v : s + v;
            if (q % L == L - 1) y = (q / L == 0) ? s : y + s;
        }
        return y;
    }
}

// Two element groups at once (all 2*W loads issued before any add).
template <int WT, int LT, class LD>
__device__ __forceinline__ void ordered_sum2(const LD &ld, int64_t idx, int64_t idx2,
                                             int64_t stride, int W, int L_rt, f32x4_t *y_out,
                                             f32x4_t *y2_out) {
    const int L = LT > 0 ? LT : L_rt;
    if constexpr (WT > 0) {
        f32x4_t v[WT], u[WT];
#pragma unroll
        for (int q = 0; q < WT; ++q) {
            v[q] = ld(idx + q * stride);
            u[q] = ld(idx2 + q * stride);
        }
        f32x4_t y = v[0], s = v[0], y2 = u[0], s2 = u[0];
#pragma unroll
        for (int q = 0; q < WT; ++q) {
            s = (q % L == 0) ? v[q] : s + v[q];
            s2 = (q % L == 0) ? u[q] : s2 + u[q];
            if (q % L == L - 1) {
                y = (q / L == 0) ? s : y + s;
                y2 = (q / L == 0) ? s2 : y2 + s2;
            }
        }
        *y_out = y;
        *y2_out = y2;
    } else {
        *y_out = ordered_sum<0, LT>(ld, idx, stride, W, L);
        *y2_out = ordered_sum<0, LT>(ld, idx2, stride, W, L);
    }
}

// Tile and slab of this workgroup.  kSliceAll: unit = t*U + slab.
// kSliceSteps: unit = (k - k_lo)*U + slab names the k-th tile of the order
// every rank shares (rank 0's k-th tile).
__device__ __forceinline__ void unit_tile(const ReduceArgs &a, int32_t *t, int32_t *slab) {
    const TileGeom &g = a.g;
    const uint32_t U = (uint32_t)a.units_per_tile, unit = blockIdx.x;
    *slab = (int32_t)(unit % U);
    const uint32_t rest = unit / U, W = (uint32_t)g.W;
    int32_t r;
    if (a.slice_kind == kSliceAll) {
        *t = (int32_t)rest;
        return;
    }
    tile_of_block(g, (a.k_lo + rest) * W, &r, t);
}

// One-stage reduce: flags -> out.  ROWS2: two rows per thread and
// iteration (2*W loads in flight); without it one row (W loads, fewer
// registers: the slices that run beside the GEMM must fit in the registers
// its workgroups leave free).  Both sum in the same order.
template <int WT, int LT, bool OUT_BF16, bool SB, bool ROWS2, bool BUF>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
    const TileGeom &g = a.g;
    const int32_t U = a.units_per_tile;
    int32_t t, slab;
    unit_tile(a, &t, &slab);
    const int32_t tm = t / g.tiles_n, tn = t - (t / g.tiles_n) * g.tiles_n;

    if (!wait_flags(a.flags + t, g.T, g.W, a.timeout_ticks, a.err, 0, t)) return;
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(&a.counters[t], 1u);
        if (old == (uint32_t)U - 1) {   // every unit of the tile has passed
            if (!a.keep_flags)
                for (int q = 0; q < g.W; ++q)
                    __hip_atomic_store(&a.flags[(int64_t)q * g.T + t], 0u,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.counters[t], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    int64_t lo, hi;
    unit_rows(g, tm, slab, &lo, &hi);
    const int W = g.W, L = W / a.groups;
    const int C4 = g.BN / 4;                  // float4 per tile row
    const int RPP = kThreads / C4;            // rows per pass
    const int c4 = threadIdx.x % C4;
    const int64_t col = (int64_t)tn * g.BN + c4 * 4;
    const int64_t stride = g.slot;
    auto sum_rows = [&](const auto &ld) __attribute__((always_inline)) {
        if constexpr (!ROWS2) {
            for (int64_t row = lo + threadIdx.x / C4; row < hi; row += RPP) {
                const int64_t d = row / g.Mc;
                const int64_t idx = (d * W) * g.slot + (row - d * g.Mc) * g.N + col;
                store_out4(a.out, row * g.N + col, ordered_sum<WT, LT>(ld, idx, stride, W, L),
                           OUT_BF16);
            }
            return;
        }
        // two rows per thread per iteration: 2*W independent 16-byte loads
        for (int64_t row = lo + threadIdx.x / C4; row < hi; row += 2 * RPP) {
            const int64_t row2 = row + RPP;
            const int64_t d = row / g.Mc;
            const int64_t idx = (d * W) * g.slot + (row - d * g.Mc) * g.N + col;
            if (row2 < hi) {
                const int64_t d2 = row2 / g.Mc;
                const int64_t idx2 = (d2 * W) * g.slot + (row2 - d2 * g.Mc) * g.N + col;
                f32x4_t y, y2;
                ordered_sum2<WT, LT>(ld, idx, idx2, stride, W, L, &y, &y2);
                store_out4(a.out, row * g.N + col, y, OUT_BF16);
                store_out4(a.out, row2 * g.N + col, y2, OUT_BF16);
            } else {
                store_out4(a.out, row * g.N + col, ordered_sum<WT, LT>(ld, idx, stride, W, L),
                           OUT_BF16);
            }
        }
    };
    if constexpr (BUF) sum_rows(BufSlots(a.staging, a.staging_bytes));
    else sum_rows(PtrSlots<SB>{a.staging});
}

// Materialised two-level, stage 1: group g's partial sum -> sub buffer.
template <int LT>
__global__ __launch_bounds__(kThreads) void reduce_sub_kernel(ReduceArgs a) {
    const TileGeom &g = a.g;
    const int32_t U = a.units_per_tile, G = a.groups, L = g.W / G;
    const int64_t per_group = (int64_t)g.T * U;
    const int32_t grp = (int32_t)(blockIdx.x / per_group);
    const int64_t unit = blockIdx.x - (int64_t)grp * per_group;
    const int32_t t = (int32_t)(unit / U), slab = (int32_t)(unit % U);
    const int32_t tm = t / g.tiles_n, tn = t - (t / g.tiles_n) * g.tiles_n;

    if (!wait_flags(a.flags + (int64_t)grp * L * g.T + t, g.T, L,
                    a.timeout_ticks, a.err, grp * L, t))
        return;
    if (threadIdx.x == 0) {
        uint32_t *cnt = &a.counters[(int64_t)grp * g.T + t];
        const uint32_t old = atomicAdd(cnt, 1u);
        if (old == (uint32_t)U - 1) {
            if (!a.keep_flags)
                for (int q = 0; q < L; ++q)
                    __hip_atomic_store(&a.flags[(int64_t)(grp * L + q) * g.T + t], 0u,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    int64_t lo, hi;
    unit_rows(g, tm, slab, &lo, &hi);
    const int C4 = g.BN / 4;
    const int64_t n4 = (hi - lo) * C4;
    const int64_t stride = g.slot;
    for (int64_t e = threadIdx.x; e < n4; e += kThreads) {
        const int64_t row = lo + e / C4;
        const int64_t col = (int64_t)tn * g.BN + (e % C4) * 4;
        const int64_t d = row / g.Mc, il = row - d * g.Mc;
        const int64_t idx = (d * g.W + (int64_t)grp * L) * g.slot + il * g.N + col;
        const f32x4_t s = ordered_sum<LT, LT>(PtrSlots<false>{a.staging}, idx, stride, L, L);
        float *dst = a.sub + ((d * G + grp) * g.Mc + il) * g.N + col;
        __builtin_nontemporal_store(s, (f32x4_t *)dst);
    }
    // the consumer (the final stage) runs in the next launch on the stream,
    // whose boundary makes these stores visible: the sub-flag is a plain
    // store after the workgroup's stores
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.sub_flags[(int64_t)grp * per_group + unit], 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Materialised two-level, stage 2: y = ((S_0 + S_1) + ...) -> out.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void reduce_final_sub_kernel(ReduceArgs a) {
    const TileGeom &g = a.g;
    const int32_t U = a.units_per_tile, G = a.groups;
    const int64_t per_group = (int64_t)g.T * U;
    const int64_t unit = blockIdx.x;
    const int32_t t = (int32_t)(unit / U), slab = (int32_t)(unit % U);
    const int32_t tm = t / g.tiles_n, tn = t - (t / g.tiles_n) * g.tiles_n;

    if (!wait_flags(a.sub_flags + unit, per_group, G, a.timeout_ticks,
                    a.err, 0, t))
        return;
    // a sub-flag has exactly one consumer: reset it right after the wait
    if (threadIdx.x < G && !a.keep_flags)
        __hip_atomic_store(&a.sub_flags[(int64_t)threadIdx.x * per_group + unit], 0u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    int64_t lo, hi;
    unit_rows(g, tm, slab, &lo, &hi);
    const int C4 = g.BN / 4;
    const int64_t n4 = (hi - lo) * C4;
    const int64_t stride = g.Mc * g.N;
    for (int64_t e = threadIdx.x; e < n4; e += kThreads) {
        const int64_t row = lo + e / C4;
        const int64_t col = (int64_t)tn * g.BN + (e % C4) * 4;
        const int64_t d = row / g.Mc, il = row - d * g.Mc;
        const int64_t idx = ((d * G) * g.Mc + il) * g.N + col;
        const f32x4_t y = ordered_sum<0, 0>(PtrSlots<false>{a.sub}, idx, stride, G, G);
        store_out4(a.out, row * g.N + col, y, OUT_BF16);
    }
}

// Zero two word ranges (flags and counters, and an error record) with a
// kernel rather than a memset, so the enqueue stays capturable in a graph.
__global__ void clear_words_kernel(uint32_t *a, int64_t na, uint32_t *b, int64_t nb) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < na) a[i] = 0u;
    else if (i < na + nb) b[i - na] = 0u;
}

__global__ void slot_table_kernel(TileGeom g, uint32_t *tab) {
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t n = (uint32_t)g.W * (uint32_t)g.T;
    if (h >= n) return;
    int32_t r, t;
    tile_of_block(g, logical_block(g, 0, n, (uint32_t)h), &r, &t);
    tab[h] = ((uint32_t)r << kSlotTileBits) | (uint32_t)t;
}

__global__ void tile_order_kernel(TileGeom g, int32_t *trace) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= (int64_t)g.W * g.T) return;
    int32_t r, t;
    tile_of_block(g, (uint32_t)b, &r, &t);
    trace[b] = t;
}

// W unrolled for 1, 2, 4 and 8 slots; the group length at compile time
// for the flat order (L = W) and two groups (L = W/2).
template <int WT, bool BF, bool SB, bool ROWS2, bool BUF>
void launch_wl(const ReduceArgs &a, dim3 grid, hipStream_t s) {
    const int L = a.g.W / a.groups;
    if constexpr (WT > 0) {
        if (L == WT) {
            hipLaunchKernelGGL((reduce_kernel<WT, WT, BF, SB, ROWS2, BUF>), grid, dim3(kThreads), 0,
                               s, a);
            return;
        }
        if constexpr (WT >= 2) {
            if (L == WT / 2) {
                hipLaunchKernelGGL((reduce_kernel<WT, WT / 2, BF, SB, ROWS2, BUF>), grid,
                                   dim3(kThreads), 0, s, a);
                return;
            }
        }
    }
    hipLaunchKernelGGL((reduce_kernel<WT, 0, BF, SB, ROWS2, BUF>), grid, dim3(kThreads), 0, s, a);
}

template <bool BF, bool SB, bool ROWS2, bool BUF>
hipError_t launch_w(const ReduceArgs &a, dim3 grid, hipStream_t s) {
    switch (a.g.W) {
    case 1: launch_wl<1, BF, SB, ROWS2, BUF>(a, grid, s); break;
    case 2: launch_wl<2, BF, SB, ROWS2, BUF>(a, grid, s); break;
    case 4: launch_wl<4, BF, SB, ROWS2, BUF>(a, grid, s); break;
    case 8: launch_wl<8, BF, SB, ROWS2, BUF>(a, grid, s); break;
    default: launch_wl<0, BF, SB, ROWS2, BUF>(a, grid, s); break;
    }
    return hipGetLastError();
}

template <bool BF, bool SB>
hipError_t launch_flat(const ReduceArgs &a, hipStream_t s) {
    const int64_t units = a.slice_kind == kSliceSteps
                              ? (int64_t)(a.k_hi - a.k_lo) * a.units_per_tile
                              : (int64_t)a.g.T * a.units_per_tile;
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)units);
    // slices run beside GEMM launches: the one-row form
    if (a.slice_kind != kSliceAll) return launch_w<BF, SB, false, false>(a, grid, s);
    // fp32 staging below 4 GiB: the slots through one buffer descriptor
    if constexpr (!SB)
        if (a.staging_bytes <= (int64_t)0xffffffffu)
            return launch_w<BF, SB, true, true>(a, grid, s);
    return launch_w<BF, SB, true, false>(a, grid, s);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, int dtype, hipStream_t s) {
    if (dtype != GEMM_RS_BF16) return launch_flat<false, false>(a, s);
    return a.staging_bf16 ? launch_flat<true, true>(a, s) : launch_flat<true, false>(a, s);
}

hipError_t launch_reduce_sub(const ReduceArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.groups * a.g.T * a.units_per_tile));
    const int L = a.g.W / a.groups;
    switch (L) {
    case 4: hipLaunchKernelGGL((reduce_sub_kernel<4>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((reduce_sub_kernel<0>), grid, dim3(kThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_reduce_final_sub(const ReduceArgs &a, int dtype, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.g.T * a.units_per_tile));
    if (dtype == GEMM_RS_BF16)
        hipLaunchKernelGGL((reduce_final_sub_kernel<true>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((reduce_final_sub_kernel<false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_clear_words(uint32_t *a, int64_t na, uint32_t *b, int64_t nb,
                              hipStream_t s) {
    const int64_t n = na + nb;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a, na, b, nb);
    return hipGetLastError();
}

hipError_t launch_slot_table(const TileGeom &g, uint32_t *tab, hipStream_t s) {
    const int64_t n = (int64_t)g.W * g.T;
    hipLaunchKernelGGL(slot_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       g, tab);
    return hipGetLastError();
}

hipError_t launch_tile_order(const TileGeom &g, int32_t *trace, hipStream_t s) {
    const int64_t n = (int64_t)g.W * g.T;
    hipLaunchKernelGGL(tile_order_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       g, trace);
    return hipGetLastError();
}

}  // namespace gemm_rs
