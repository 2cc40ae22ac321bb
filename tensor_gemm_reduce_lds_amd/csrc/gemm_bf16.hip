// bf16 GEMM + reduce-scatter epilogue for gfx950.
//
// Workgroup b computes one BM x BN output tile of rank r = b % W (tile
// order: tile_of_block).
//
// Mainloop, per BK-deep K step:
//   * A[BM][BK] and B[BK][BN] tiles go from HBM straight into LDS with
//     16-byte buffer loads to LDS (no register staging) into a ring of STAGES
//     LDS stages; loads run STAGES-1 steps ahead of the MFMAs.  The DMA is
//     issued from inline asm and its completion tracked by explicit vmcnt
//     waits, so the compiler does not serialise LDS reads of one stage
//     behind DMA still in flight into another.  With 8 waves only one
//     wave per SIMD issues it, so the other wave of each SIMD only feeds
//     the matrix pipe.
//   * A sits in LDS as [m][k] rows of 2*BK bytes; B stays row-major [k][n]
//     as it is in memory; LDS holds every stage's A tile, then every
//     stage's B tile.  Both are XOR-swizzled at 16-byte granularity
//     (the swizzle is applied by choosing which global chunk each lane
//     fetches, since a DMA load writes lane l at base + 16*l).
//   * A operands come from ds_read_b128; B operands from two
//     ds_read_b64_tr_b16 per MFMA, which transpose 4x16 bf16 blocks across
//     16 lanes so that each lane gets 4 consecutive k of one column.
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulators; the LDS reads of the
//     next 16-deep slice are interleaved with the MFMAs of the current one,
//     and each step's last slice is issued after the next step's barrier.
// Epilogue: alpha*acc, plus beta*C on rows whose chunk this rank owns,
// stored as fp32 (or, optionally, rounded to bf16) into the staging slot
// of each row's destination chunk
// (rows pass through LDS so that each store instruction writes whole
// staging rows); then the tile's ready flag is published (page "flux实现：
// sm80 gemm+rs", section "cutlass自定义epilogue–sm80": a compute node
// alpha*acc + beta*C, a store node that scatters by destination, and a
// per-tile flag).  The FW instantiation also sums tiles in place of the
// separate reduce: the owner-fused last step and the last-arriver launch.
#include <mutex>
#include <type_traits>

#include "gemm_rs_internal.h"

namespace gemm_rs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

#pragma clang diagnostic ignored "-Winline-asm"

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (gfx9 layout): 48-bit base, stride 0, `bytes`
// records, 32-bit untyped data format.  A load at an offset of `bytes` or
// more returns zeros instead of touching memory.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t p = (uint64_t)base;
    i32x4_t r;
    r[0] = (int32_t)(uint32_t)p;
    r[1] = (int32_t)((uint32_t)(p >> 32) & 0xffffu);
    r[2] = (int32_t)bytes;
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from global memory straight into LDS: lane l reads
// the buffer at its byte offset `voff` and its data lands at
// lds_base + 16*l (lds_base is wave-uniform, passed in M0).  The buffer
// form takes a 32-bit offset per lane instead of a 64-bit address, half the
// address traffic of the global form (measured +3.5% on the whole GEMM).
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_base) : "memory", "m0");
}

// Cache policy of a buffer access: nt (streaming) and sc1 (device scope:
// the store is written through this XCD's L2).
constexpr int kPolicyNtSc1 = 2 | 16;

// Four bfloat16 values (lo holds the first two, low half first) widened
// exactly to floats: a bfloat16 is the top half of a float.
__device__ __forceinline__ f32x4_t widen_bf16x4(uint32_t lo, uint32_t hi) {
    f32x4_t v;
    v[0] = __uint_as_float(lo << 16);
    v[1] = __uint_as_float(lo & 0xffff0000u);
    v[2] = __uint_as_float(hi << 16);
    v[3] = __uint_as_float(hi & 0xffff0000u);
    return v;
}

// Four floats rounded to bfloat16 (nearest even), packed in the same layout.
__device__ __forceinline__ u32x2_t pack_bf16x4(f32x4_t x) {
    const __bf16 h0 = (__bf16)x[0], h1 = (__bf16)x[1];
    const __bf16 h2 = (__bf16)x[2], h3 = (__bf16)x[3];
    u32x2_t w;
    w[0] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
           ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    w[1] = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
           ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
    return w;
}

// A workgroup barrier for LDS hand-offs only: it waits for this wave's LDS
// operations but not for its global stores, which __syncthreads would also
// drain (its release fence covers global memory), a full memory latency.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait until at most `pending` DMA groups of `per` loads are in flight.
template <int PER, int MAXP>
__device__ __forceinline__ void wait_groups(int pending) {
    if constexpr (MAXP >= 3) { if (pending >= 3) { wait_vmcnt<3 * PER>(); return; } }
    if constexpr (MAXP >= 2) { if (pending >= 2) { wait_vmcnt<2 * PER>(); return; } }
    if constexpr (MAXP >= 1) { if (pending >= 1) { wait_vmcnt<PER>(); return; } }
    wait_vmcnt<0>();
}

// A rows are 2*BK bytes (BK/8 chunks of 16 bytes); chunk c of row m lives
// at c ^ swa(m).  The 16 rows read by 16 lanes then cover all 64 banks once.
template <int BK>
__device__ __forceinline__ int swa(int m) {
    if constexpr (BK == 64) return (m ^ (m >> 3)) & 7;
    else return (m >> 2) & 3;
}
// B rows: chunk c of row k lives at c ^ swb(k).  A transpose read touches
// 4 consecutive k rows x 4 chunks per 32 lanes; XOR with 4*(k%4) spreads
// them over 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swb(int k) { return 4 * (k & 3); }

// FW > 0: the owner-fused reduce variant for W == FW ranks (see GemmArgs).
// U2: the K loop unrolled by two steps, so that each step's stage is a
// compile-time constant and its fragment reads take the stage offset in their
// immediate field (no per-read address add; ~1% at the 70B-like shard).  It
// needs every register of two waves per SIMD, so launches that must leave
// room for other kernels' waves on the same CUs (the all-gather's copies,
// the identity-order reduce slices) use the rolled loop.
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int FW, bool U2>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int NW = WGM * WGN;                 // waves
    constexpr int WM = BM / WGM, WN = BN / WGN;   // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 blocks per wave
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    // LDS holds the A tiles of all stages, then the B tiles of all stages:
    // stage s of an operand lies s tiles past its first, an offset that fits
    // a DS read's 16-bit immediate, so with the stage known at compile time
    // the fragment reads need no per-read address add
    constexpr int B_REGION = STAGES * A_BYTES;
    constexpr int A_ISSUES = A_BYTES / 1024 / NW;  // 1 KB DMA loads per wave
    constexpr int B_ISSUES = B_BYTES / 1024 / NW;
    constexpr int CPA = BK / 8;                   // 16-byte chunks per A row
    constexpr int A_ROWS = 1024 / (BK * 2);       // A rows per 1 KB
    constexpr int CPR = BN / 8;                   // 16-byte chunks per B row
    constexpr int B_ROWS = 1024 / (BN * 2);       // B rows per 1 KB
    static_assert(A_ISSUES * NW * 1024 == A_BYTES && B_ISSUES * NW * 1024 == B_BYTES, "");
    static_assert(CPR >= 16, "B swizzle needs rows of at least 16 chunks");

    extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
    lds_char *smem = (lds_char *)smem_generic;
    const uint32_t smem_base = (uint32_t)(size_t)smem;

    const TileGeom &g = a.g;
    int32_t r, t;
    uint32_t b;
    if (a.slot_tab) {
        // the full launch: the slot's rank and tile were tabulated with the
        // plan (one scalar load instead of the tile-order arithmetic, which
        // every wave of the workgroup would repeat on the shared scalar unit)
        const uint32_t v = a.slot_tab[blockIdx.x];
        r = (int32_t)(v >> kSlotTileBits);
        t = (int32_t)(v & ((1u << kSlotTileBits) - 1u));
        b = a.trace ? logical_block(g, 0, a.n_blocks, blockIdx.x) : 0u;   // trace index only
    } else {
        b = a.xcd_rank_major ? logical_block(g, a.b_offset, a.n_blocks, blockIdx.x)
                             : a.b_offset + blockIdx.x;
        tile_of_block(g, b, &r, &t);
    }
    const int32_t tm = t / g.tiles_n, tn = t - (t / g.tiles_n) * g.tiles_n;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    // (the unrolled instantiation is never launched gated: without the
    // gate's workgroup vote it holds no static LDS, its dynamic LDS starts
    // at address 0, and every fragment address folds into the reads'
    // immediate offsets)
    if constexpr (!U2) if (a.signals) {
        // all-gather mode: wait until this tile-row of A has been copied in
        // (agent-scope acquire, bounded); the loads below then see it
        int failed = 0;
        if (tid == 0) {
            const uint32_t *sig = a.signals + (int64_t)r * g.tiles_m + tm;
            const uint64_t t0 = wall_clock64();
            while (__hip_atomic_load(sig, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) !=
                   a.epoch) {
                if (wall_clock64() - t0 > a.timeout_ticks) {
                    failed = 1;
                    record_error(a.err, GEMM_RS_ERR_TIMEOUT, r, tm, 0);
                    break;
                }
                __builtin_amdgcn_s_sleep(4);
            }
        }
        if (__syncthreads_or(failed)) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }

    const uint16_t *A = (const uint16_t *)a.A + (int64_t)r * g.M * g.K;
    const uint16_t *B = (const uint16_t *)a.B + (int64_t)r * g.K * g.N;
    const int64_t row0 = (int64_t)tm * BM, col0 = (int64_t)tn * BN;

    // ---- per-lane DMA byte offsets inside one K step's windows ----
    // Step kt reads the A window (the tile's rows, columns [kt*BK, +BK))
    // from a descriptor based at A[row0][kt*BK] and the B window (rows
    // [kt*BK, +BK), the tile's columns) from one based at B[kt*BK][col0];
    // the per-lane offsets stay the same every step and fit 32 bits
    // (K < 2^23, N < 2^25: plan limits).
    const int64_t a_rows = g.M - row0 < BM ? g.M - row0 : BM;
    const uint32_t a_bytes = (uint32_t)(((a_rows - 1) * g.K + BK) * 2);
    const uint32_t b_bytes = (uint32_t)(((int64_t)(BK - 1) * g.N + BN) * 2);
    // With 8 waves the operand DMA is issued by waves 0..3 only, one per
    // SIMD (wave w runs on SIMD w % 4), each with twice the loads: every
    // SIMD then has one wave that only reads LDS fragments and issues
    // MFMAs, which keeps the matrix pipe fed while the other wave issues
    // the DMA (measured +3% on the 70B-like shard, +2-6% on the 8B-like).
    constexpr int DW = NW >= 8 ? NW / 2 : NW;     // waves that issue the DMA
    constexpr int AI = A_ISSUES * NW / DW, BI = B_ISSUES * NW / DW;
    static_assert(AI * DW == A_ISSUES * NW && BI * DW == B_ISSUES * NW, "");
    const int dwave = wave < DW ? wave : 0;
    uint32_t a_voff[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int m = (i * DW + dwave) * A_ROWS + lane / CPA;
        const int64_t ml = m < a_rows ? m : a_rows - 1;   // ragged M: fetch a valid row
        a_voff[i] = (uint32_t)((ml * g.K + ((lane % CPA) ^ swa<BK>(m)) * 8) * 2);
    }
    uint32_t b_voff[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int k = (i * DW + dwave) * B_ROWS + lane / CPR;
        b_voff[i] = (uint32_t)(((int64_t)k * g.N + ((lane % CPR) ^ swb(k)) * 8) * 2);
    }

    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
        if (wave >= DW) return;                     // wave-uniform
        const uint32_t As = smem_base + buf * A_BYTES;
        const uint32_t Bs = smem_base + B_REGION + buf * B_BYTES;
        const i32x4_t a_rsrc = buffer_rsrc(A + row0 * g.K + (int64_t)kt * BK, a_bytes);
        const i32x4_t b_rsrc = buffer_rsrc(B + (int64_t)kt * BK * g.N + col0, b_bytes);
#pragma unroll
        for (int i = 0; i < AI; ++i)
            dma16(a_rsrc, a_voff[i], As + (i * DW + dwave) * 1024);
#pragma unroll
        for (int i = 0; i < BI; ++i)
            dma16(b_rsrc, b_voff[i], Bs + (i * DW + dwave) * 1024);
    };

    // ---- per-lane LDS read offsets (bytes, within a stage) ----
    int a_off[FM][BK / 16];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int m = wm * WM + i * 32 + (lane & 31);
            const int c = 2 * ks + (lane >> 5);
            a_off[i][ks] = m * (BK * 2) + ((c ^ swa<BK>(m)) << 4);
        }
    // transpose-read source lane: row kbase + e, columns 4q..4q+3 of its
    // 16-column group (e = (lane%16)/4, q = lane%4)
    int b_off[FN][BK / 16][2];
    {
        const int grp = lane >> 4, i16 = lane & 15;
        const int e = i16 >> 2, q = i16 & 3;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = ks * 16 + 8 * (grp >> 1) + 4 * h + e;
                    const int n = wn * WN + j * 32 + 16 * (grp & 1) + 4 * q;
                    b_off[j][ks][h] = B_REGION + k * (BN * 2) +
                                      (((n >> 3) ^ swb(k)) << 4) + ((n & 7) << 1);
                }
    }

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto load_frags = [&](int st, int ks, bf16x8_t (&af)[FM], bf16x8_t (&bfr)[FN])
        __attribute__((always_inline)) {
        lds_char *const SA = smem + st * A_BYTES, *const SB = smem + st * B_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *(__attribute__((address_space(3))) bf16x8_t *)(SA + a_off[i][ks]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(SB + b_off[j][ks][0]));
            i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(SB + b_off[j][ks][1]));
            i16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            bfr[j] = __builtin_bit_cast(bf16x8_t, both);
        }
    };
    // Operand fragments are double-buffered in registers: the LDS reads of
    // the next 16-deep slice are interleaved one by one with the MFMAs of
    // the current slice, so their latency hides behind the matrix pipe.
    // Each step's last slice is issued after the next step's barrier: its
    // fragments are already in registers, and its MFMAs cover the latency
    // of the next step's first reads, so the matrix pipes do not drain at
    // every barrier.
    constexpr int KS = BK / 16;
    static_assert(KS % 2 == 0, "the last slice uses fragment buffer 1");
    bf16x8_t af[2][FM], bfr[2][FN];
    auto mfmas = [&](int fb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                // operands swapped: the block comes out transposed, so a
                // lane holds one output row and runs of 4 columns
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    bfr[fb][j], af[fb][i], acc[i][j], 0, 0, 0);
    };
    auto interleave = [&]() __attribute__((always_inline)) {
        // schedule: one LDS read (mask 0x100), one MFMA (0x008), ...
#pragma unroll
        for (int k = 0; k < FM + 2 * FN; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    };

    const int KT = (int)(g.K / BK);
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) issue(s, s);
    // the bias row of the tile's columns (ldc == 0): one 8-byte load per
    // lane, issued with the first operand loads, so it has arrived by the
    // epilogue; the unrolled loop has no registers to hold it across the
    // mainloop (it would be spilled), so there it is loaded after the loop,
    // ahead of the last MFMA slice
    uint2 cb_row = {0u, 0u};
    if constexpr (!U2)
        if (a.has_c && a.ldc == 0)
            cb_row = *(const uint2 *)((const uint16_t *)a.C + col0 + (lane % (BN / 4)) * 4);
    if constexpr (FW > 0) if (a.fuse_reduce == kFuseOwner) {
        // owner-fused reduce: every other rank's partial of this tile was
        // staged by an earlier launch on the stream (so it is visible
        // here); its flag must read 1.  Checked while the first operand
        // loads are in flight, then every flag of the tile is put back to
        // 0 (this rank's own never left it): this workgroup is the tile's
        // only consumer, and the flags end the run idle as after the
        // separate reduce.
        int failed = 0;
        if (tid < FW && tid != r)
            failed = wait_flag_set(a.flags + (int64_t)tid * g.T + t, a.timeout_ticks, a.err,
                                   tid, t);
        if (__syncthreads_or(failed)) {
            wait_vmcnt<0>();                        // no DMA into LDS after exit
            return;
        }
        if (tid < FW)
            __hip_atomic_store(a.flags + (int64_t)tid * g.T + t, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    static_assert(STAGES == 2, "steps alternate between two stages");
    auto step = [&](int kt, auto st_tag) __attribute__((always_inline)) {
        const int ST = st_tag;   // kt % 2: a compile-time constant or a run-time value
        // wait until this wave's DMA for step kt has landed (later steps
        // may stay in flight); the barrier makes every wave's data visible
        // and frees the stage read in step kt-1 for the next issue
        const int ahead = KT - 1 - kt;
        wait_groups<AI + BI, STAGES - 2>(ahead < STAGES - 2 ? ahead : STAGES - 2);
        __syncthreads();
        load_frags(ST, 0, af[0], bfr[0]);
        if (kt > 0) mfmas(1);   // the previous step's last slice
        if (kt + 1 < KT) issue(kt + 1, 1 - ST);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            load_frags(ST, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
            mfmas(ks & 1);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (U2) {
        int kt = 0;
        for (; kt + 1 < KT; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }
        if (kt < KT) step(kt, std::integral_constant<int, 0>{});
    } else {
        for (int kt = 0; kt < KT; ++kt) step(kt, kt & 1);
    }
    if constexpr (U2)
        if (a.has_c && a.ldc == 0)
            cb_row = *(const uint2 *)((const uint16_t *)a.C + col0 + (lane % (BN / 4)) * 4);
    if (KT > 0) mfmas(1);   // the last step's last slice

    // ---- epilogue: D = alpha*acc (+ beta*C on owned rows), scatter ----
    // beta*C is added with one fused multiply-add, in every path (plain,
    // ragged and fused epilogues), so all of them round a staged value alike.
    // The accumulators go out through LDS one 32-row stripe at a time so
    // that every store instruction writes whole staging rows (64 lanes x
    // 16 bytes = 1 KB contiguous for BN = 256): a store pattern of 32 rows x
    // 32 bytes per instruction drains several times slower per CU.
    // Transposed 32x32 accumulator layout: lane holds output row (lane & 31)
    // of the block; registers 4q..4q+3 hold its columns 8q + 4*(lane/32)
    // + 0..3.
    constexpr int EP_PITCH = BN * 4 + 16;          // bytes per staged row (padded; fused epilogue)
    constexpr int LPR = BN / 4;                    // lanes per row (16 bytes each)
    constexpr int RPI = 64 / LPR;                  // rows per store instruction
    constexpr int SROWS = WGM * 32;                // rows per stripe
    constexpr int ST_PER_WAVE = SROWS / (NW * RPI);
    static_assert(SROWS * EP_PITCH <= STAGES * STAGE, "stripe fits in the stage buffers");
    static_assert(ST_PER_WAVE * NW * RPI == SROWS, "stripe rows split evenly");
    static_assert(32 % (ST_PER_WAVE * RPI) == 0, "a wave's stripe rows stay in one 32-row group");
    // The plain epilogue's stripes alternate between the two stages, with
    // rows of BN*4 bytes whose 16-byte chunk c of row rr sits at c ^ (rr %
    // 16): the 16 rows one write covers and the chunks one read covers both
    // land on distinct banks without padding, so a stripe fits one stage
    // (its A tile, then its B tile).
    // The stage that held step KT-2 is free on arrival (every wave has
    // passed the barrier that followed its last reads of it), so the first
    // stripe needs no barrier before it; the stage of step KT-1 is free
    // once every wave has passed the first stripe's barrier.
    constexpr int EP_ROW = BN * 4;
    static_assert(SROWS * EP_ROW <= STAGE, "a stripe fits one stage");
    static_assert(STAGES == 2, "stripes alternate between the two stages");
    // a stripe in stage s: its first A_BYTES / EP_ROW rows in the stage's A
    // tile, the rest in its B tile
    constexpr int ROWS_IN_A = A_BYTES / EP_ROW;
    static_assert(ROWS_IN_A * EP_ROW == A_BYTES, "");
    const int ep_st[2] = {KT & 1, (KT + 1) & 1};
    const uint16_t *Cp = (const uint16_t *)a.C;
    const float alpha = a.alpha, beta = a.beta;
    const int h4 = 4 * (lane >> 5);
    const int scol = (lane % LPR) * 4;              // this lane's 4 columns in a row
    const int srow = lane / LPR;                    // row inside a store instruction
    // C modes: 0 none, 1 bias row (ldc == 0: one 8-byte load per lane for
    // the whole tile), 2 full matrix (the stripe's rows are loaded before
    // its stores).  Each mode is separate code: a C load issued behind
    // stores would have to wait for all of them (memory operations complete
    // in order), so no load sits between two stores.
    // one staged row piece: a streaming store, or with stage_wt (the
    // last-arriver launch, FW > 0 only) a streaming device-scope buffer
    // store through the staging descriptor
    auto stage_store = [&](f32x4_t x, float *dst) __attribute__((always_inline)) {
        bool wt = false;
        if constexpr (FW > 0) wt = a.stage_wt != 0;
        if (wt) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                a.staging, (short)0, (int)(uint32_t)a.staging_bytes, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, x), rs,
                (int)(uint32_t)((const char *)dst - (const char *)a.staging), 0, kPolicyNtSc1);
        } else {
            __builtin_nontemporal_store(x, (f32x4_t *)dst);
        }
    };
    auto epilogue = [&](auto mode_tag) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_tag)::value;
        // the bias row's 4 columns, widened
        const f32x4_t cf = MODE == 1 ? widen_bf16x4(cb_row.x, cb_row.y) : f32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            // stage block i of every wave: stripe rows wm*32 .. +31 hold tile
            // rows wm*WM + i*32 .. +31 across all BN columns
            const int est = ep_st[i & 1];
            // stripe row sr, columns 4c .. 4c+3
            auto at = [&](int sr, int c) __attribute__((always_inline)) {
                lds_char *const row = sr < ROWS_IN_A
                                          ? smem + est * A_BYTES + sr * EP_ROW
                                          : smem + B_REGION + est * B_BYTES +
                                                (sr - ROWS_IN_A) * EP_ROW;
                return (__attribute__((address_space(3))) f32x4_t *)(
                    row + ((c ^ (sr & 15)) << 4));
            };
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4_t x;
#pragma unroll
                    for (int u = 0; u < 4; ++u) x[u] = alpha * acc[i][j][4 * q + u];
                    *at(wm * 32 + (lane & 31), (wn * WN + j * 32 + 8 * q + h4) >> 2) = x;
                }
            uint2 cb_full[ST_PER_WAVE];
            if constexpr (MODE == 2) {
#pragma unroll
                for (int k = 0; k < ST_PER_WAVE; ++k) {
                    const int sr = (wave * ST_PER_WAVE + k) * RPI + srow;
                    int64_t row = row0 + (sr >> 5) * WM + i * 32 + (sr & 31);
                    if (row > g.M - 1) row = g.M - 1;   // ragged M: a valid row
                    cb_full[k] = *(const uint2 *)(Cp + row * a.ldc + col0 + scol);
                }
#pragma unroll
                for (int k = 0; k < ST_PER_WAVE; ++k)   // one wait, before any store
                    asm volatile("" : "+v"(cb_full[k].x), "+v"(cb_full[k].y));
            }
            lds_barrier();                          // the stripe is in LDS
            // this lane's rows in the stripe are rowF + k*RPI (one 32-row
            // group per wave), so the destination offset is computed once
            // and advanced by RPI rows per store; only a row that crosses
            // into the next chunk recomputes it
            const int sr0 = wave * ST_PER_WAVE * RPI + srow;
            const int64_t slot_d = (int64_t)g.W * g.slot, slot_r = (int64_t)r * g.slot;
            const int64_t rowF = row0 + (sr0 >> 5) * WM + i * 32 + (sr0 & 31);
            const int32_t dF = (int32_t)((uint64_t)rowF / (uint64_t)g.Mc);
            const int64_t next_chunk = (int64_t)(dF + 1) * g.Mc;
            const int64_t offF =
                a.plain_out ? ((int64_t)r * g.M + rowF) * g.N + col0 + scol
                            : (int64_t)dF * slot_d + slot_r + (rowF - (int64_t)dF * g.Mc) * g.N +
                                  col0 + scol;
            auto store_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int k = 0; k < ST_PER_WAVE; ++k) {
                    const int sr = sr0 + k * RPI;               // row in the stripe set
                    const int64_t row = rowF + k * RPI;
                    f32x4_t x = *at(sr, scol >> 2);
                    if (row < g.M) {
                        int32_t d = dF;
                        int64_t off = offF + (int64_t)(k * RPI) * g.N;
                        if (row >= next_chunk) {   // a chunk boundary inside the group
                            d = (int32_t)((uint64_t)row / (uint64_t)g.Mc);
                            off = a.plain_out ? ((int64_t)r * g.M + row) * g.N + col0 + scol
                                              : (int64_t)d * slot_d + slot_r +
                                                    (row - (int64_t)d * g.Mc) * g.N + col0 + scol;
                        }
                        if constexpr (MODE != 0) {
                            const uint2 cb = MODE == 1 ? cb_row : cb_full[k];
                            const f32x4_t c = widen_bf16x4(cb.x, cb.y);
                            const bool own = d == r;    // C counts once: on its owner's rows
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const float yu = __builtin_fmaf(beta, c[u], x[u]);
                                x[u] = own ? yu : x[u];
                            }
                        }
                        // whole 128-byte lines from one instruction: a streaming
                        // store keeps the staging from evicting the A/B panels
                        // other tiles are still reading
                        if (a.staging_bf16) {
                            // bfloat16 staging: each partial rounded to nearest even
                            __builtin_nontemporal_store(pack_bf16x4(x),
                                                        (u32x2_t *)((uint16_t *)a.staging + off));
                        } else {
                            stage_store(x, (float *)a.staging + off);
                        }
                    }
                }
            };
            const int64_t rowL = rowF + (int64_t)(ST_PER_WAVE - 1) * RPI;
            if constexpr (MODE != 2) {
                if (rowL < g.M && rowL < next_chunk) {
                    // the common case: every row of the group lies inside the
                    // matrix and in one chunk, so the owner test, the C term
                    // and the staging format are decided once, and each row
                    // is one LDS read, an optional add and one store
                    const bool add_c = MODE == 1 && dF == r;
                    const int64_t step = (int64_t)RPI * g.N;
                    if (a.staging_bf16) {
                        uint16_t *dst = (uint16_t *)a.staging + offF;
#pragma unroll
                        for (int k = 0; k < ST_PER_WAVE; ++k, dst += step) {
                            f32x4_t x = *at(sr0 + k * RPI, scol >> 2);
                            if (add_c)
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    x[u] = __builtin_fmaf(beta, cf[u], x[u]);
                            __builtin_nontemporal_store(pack_bf16x4(x), (u32x2_t *)dst);
                        }
                    } else {
                        float *dst = (float *)a.staging + offF;
#pragma unroll
                        for (int k = 0; k < ST_PER_WAVE; ++k, dst += step) {
                            f32x4_t x = *at(sr0 + k * RPI, scol >> 2);
                            if (add_c)
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    x[u] = __builtin_fmaf(beta, cf[u], x[u]);
                            stage_store(x, dst);
                        }
                    }
                } else {
                    store_rows();   // ragged rows or a chunk boundary inside the group
                }
            } else {
                store_rows();
            }
            // no barrier here: the next stripe goes to the other stage, and
            // the one after it waits for the next stripe's barrier, which
            // every wave reaches after its reads of this one
        }
    };
    // ---- owner-fused reduce epilogue ----
    // Rank r owns every row of this tile that lies in chunk r, and this is
    // the tile's last contribution: the other W-1 partials of each row i
    // are in staging slots (d(i), q).  Each row's W partials are summed in
    // the reduce order with this rank's own value (alpha*acc, plus beta*C on
    // rows of its own chunk, rounded as staging would hold it) at position
    // r, then rounded to bf16 and written to `out`; the own partial is
    // never staged.  The stripes pass through LDS as in the plain epilogue,
    // so a lane holds 4 consecutive columns of one row, the layout of the
    // staging slots.  Loads run one row ahead of the adds and stores.
    auto fused_epilogue = [&](auto mode_tag, auto sb_tag) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_tag)::value;
        constexpr bool SB = decltype(sb_tag)::value;
        constexpr int NR = FW > 1 ? FW - 1 : 1;      // remote partials per element
        typedef typename std::conditional<SB, u32x2_t, f32x4_t>::type raw_t;
        const int L = FW / a.groups;                 // ranks per group
        const int64_t slot = g.slot;                 // elements from slot (d,q) to (d,q+1)
        const int q_lo = r;                          // remote j < r is rank j, else j+1
        const f32x4_t cf = MODE == 1 ? widen_bf16x4(cb_row.x, cb_row.y) : f32x4_t{0, 0, 0, 0};
        __syncthreads();                            // every wave is done with the stages
        // the remote partials of one row (wave-uniform row for BN = 256)
        auto load_row = [&](int64_t base, raw_t (&v)[NR]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                const int64_t idx = base + (int64_t)(j < q_lo ? j : j + 1) * slot;
                if constexpr (SB)
                    v[j] = __builtin_nontemporal_load(
                        (const u32x2_t *)((const uint16_t *)a.staging + idx));
                else
                    v[j] = __builtin_nontemporal_load(
                        (const f32x4_t *)((const float *)a.staging + idx));
            }
        };
        auto widen = [](raw_t x) -> f32x4_t {
            if constexpr (SB) return widen_bf16x4(x[0], x[1]);
            else return x;
        };
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            lds_char *stripe = smem + wm * 32 * EP_PITCH;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4_t x;
#pragma unroll
                    for (int u = 0; u < 4; ++u) x[u] = alpha * acc[i][j][4 * q + u];
                    *(__attribute__((address_space(3))) f32x4_t *)(
                        stripe + (lane & 31) * EP_PITCH + (wn * WN + j * 32 + 8 * q + h4) * 4) = x;
                }
            lds_barrier();                          // the stripe is in LDS
            const int sr0 = wave * ST_PER_WAVE * RPI + srow;
            const int64_t rowF = row0 + (sr0 >> 5) * WM + i * 32 + (sr0 & 31);
            // row k of this lane: rowF + k*RPI; chunk and slot-0 offset per row
            auto row_base = [&](int k, int32_t *d_out) __attribute__((always_inline)) -> int64_t {
                int64_t row = rowF + (int64_t)k * RPI;
                if (row > g.M - 1) row = g.M - 1;   // ragged M: a valid row, not stored
                const int32_t d = (int32_t)((uint64_t)row / (uint64_t)g.Mc);
                *d_out = d;
                return ((int64_t)d * FW) * g.slot + (row - (int64_t)d * g.Mc) * g.N + col0 + scol;
            };
            raw_t cur[NR], nxt[NR];
            int32_t d_cur, d_nxt = 0;
            int64_t base_cur = row_base(0, &d_cur), base_nxt = 0;
            load_row(base_cur, cur);
#pragma unroll
            for (int k = 0; k < ST_PER_WAVE; ++k) {
                if (k + 1 < ST_PER_WAVE) {          // the next row's loads go out first
                    base_nxt = row_base(k + 1, &d_nxt);
                    load_row(base_nxt, nxt);
                }
                const int64_t row = rowF + (int64_t)k * RPI;
                f32x4_t x = *(__attribute__((address_space(3))) f32x4_t *)(
                    smem + (sr0 + k * RPI) * EP_PITCH + scol * 4);
                if constexpr (MODE != 0) {
                    f32x4_t c4 = cf;
                    if constexpr (MODE == 2) {
                        const int64_t crow = row < g.M ? row : g.M - 1;
                        const uint2 cb = *(const uint2 *)(Cp + crow * a.ldc + col0 + scol);
                        c4 = widen_bf16x4(cb.x, cb.y);
                    }
                    if (d_cur == r)                 // C counts once: on its owner's rows
#pragma unroll
                        for (int u = 0; u < 4; ++u) x[u] = __builtin_fmaf(beta, c4[u], x[u]);
                }
                if constexpr (SB) {
                    // the value a bfloat16 staging slot would hold
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        x[u] = (float)(__bf16)x[u];
                }
                // fixed order: y = sum over groups of (sum over ranks in the
                // group), ascending, with this rank's value at position r
                f32x4_t y = x, sg = x;
#pragma unroll
                for (int q = 0; q < FW; ++q) {
                    // rank q < r is remote partial q, rank q > r is q - 1
                    const f32x4_t lo = widen(cur[q < NR ? q : NR - 1]);
                    const f32x4_t hi = widen(cur[q > 0 ? q - 1 : 0]);
                    const f32x4_t v = q == r ? x : (q < r ? lo : hi);
                    sg = (q % L == 0) ? v : sg + v;
                    if (q % L == L - 1) y = (q / L == 0) ? sg : y + sg;
                }
                if (row < g.M) {
                    const u32x2_t w = pack_bf16x4(y);
                    // written through past this XCD's L2, as the reduce does
                    __hip_atomic_store((uint64_t *)((uint16_t *)a.out + row * g.N + col0 + scol),
                                       (uint64_t)w[0] | ((uint64_t)w[1] << 32), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                if (k + 1 < ST_PER_WAVE) {
#pragma unroll
                    for (int j = 0; j < NR; ++j) cur[j] = nxt[j];
                    d_cur = d_nxt;
                    base_cur = base_nxt;
                }
            }
            if (i + 1 < FM) lds_barrier();          // the stripe buffer is reused
        }
    };
    auto run_fused_epilogue = [&]() __attribute__((always_inline)) {
        if (a.staging_bf16) {
            if (!a.has_c) fused_epilogue(std::integral_constant<int, 0>{}, std::true_type{});
            else if (a.ldc == 0) fused_epilogue(std::integral_constant<int, 1>{}, std::true_type{});
            else fused_epilogue(std::integral_constant<int, 2>{}, std::true_type{});
        } else {
            if (!a.has_c) fused_epilogue(std::integral_constant<int, 0>{}, std::false_type{});
            else if (a.ldc == 0)
                fused_epilogue(std::integral_constant<int, 1>{}, std::false_type{});
            else fused_epilogue(std::integral_constant<int, 2>{}, std::false_type{});
        }
    };
    // the owner-fused workgroup goes straight to the fused epilogue; every
    // other one stages its partial and publishes it (one call site of each
    // epilogue, so both stay inlined)
    bool fused_now = false;
    if constexpr (FW > 0) fused_now = a.fuse_reduce == kFuseOwner;
    if (!fused_now) {
        if (!a.has_c) epilogue(std::integral_constant<int, 0>{});
        else if (a.ldc == 0) epilogue(std::integral_constant<int, 1>{});
        else epilogue(std::integral_constant<int, 2>{});

        // ---- publish: all stores of this tile, then flag[r][t] = 1 ----
        // With a consumer in the same launch (the last-arriver reduce) the
        // flag and the tile's stores are released together, by the release
        // fence ahead of the producer's count below: the fence comes after
        // the flag store, so the count orders both.  When the consumer is
        // stream-ordered after this kernel, the kernel boundary already makes
        // the stores visible and the flag is a plain store.
        if (!a.flags) {
            // all-gather mode: an ordinary output tile, no flag
        } else if (a.release_flags) {
            __syncthreads();                            // every wave's stores are done
            if (tid == 0)
                __hip_atomic_store(&a.flags[(int64_t)r * g.T + t], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            // the consumer runs after this kernel has completed, so the flag
            // needs no ordering against the other waves' stores here
            if (tid == 0)
                __hip_atomic_store(&a.flags[(int64_t)r * g.T + t], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0 && a.trace) a.trace[b] = t;

        // ---- last-arriver reduce ----
        // Each producer counts itself in on the tile's counter (an
        // agent-scope release fence, then a relaxed add, after its stores and
        // its flag); the one that completes the count is the tile's last
        // producer, so every partial of the tile is staged and released.  It
        // takes the acquire, checks and resets the tile's W flags and the
        // counter, and sums the tile as the owner-fused epilogue does (its own
        // partial from registers).  No workgroup ever waits for another, so
        // residency cannot deadlock it.
        if constexpr (FW > 0) if (a.fuse_reduce == kFuseLastArriver) {
            int last = 0;
            if (tid == 0) {
                // The release fence orders everything before it in this
                // workgroup (every wave's staging stores, by the barrier
                // above, and the flag) before the add; every add extends
                // the release sequence the last one reads, so its acquire
                // fence sees all W producers' stores and flags.  Only the
                // last producer pays the acquire (an L2 invalidate).
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                const uint32_t old = __hip_atomic_fetch_add(&a.counters[t], 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                if (old == (uint32_t)FW - 1) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    last = 1;
                }
                else if (old >= (uint32_t)FW) record_error(a.err, GEMM_RS_ERR_PROTOCOL, r, t, old);
            }
            if (!__syncthreads_or(last)) return;
            int bad = 0;
            if (tid < FW) {
                const uint32_t v = __hip_atomic_load(&a.flags[(int64_t)tid * g.T + t],
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v != 1u) {
                    record_error(a.err, GEMM_RS_ERR_PROTOCOL, tid, t, v);
                    bad = 1;
                }
            }
            if (__syncthreads_or(bad)) return;
            if (tid < FW && !a.keep_flags)
                __hip_atomic_store(&a.flags[(int64_t)tid * g.T + t], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0)
                __hip_atomic_store(&a.counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            fused_now = true;
        }
    }
    if constexpr (FW > 0) {
        if (fused_now) {
            run_fused_epilogue();
            if (tid == 0 && a.trace && a.fuse_reduce == kFuseOwner) a.trace[b] = t;
        }
    }
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int FW = 0, bool U2 = false>
hipError_t launch_tile(const GemmArgs &a, hipStream_t s) {
    constexpr size_t lds_bytes = (size_t)STAGES * (BM + BN) * BK * 2;
    static_assert(lds_bytes <= 160 * 1024, "LDS");
    // the dynamic LDS limit is a per-device attribute of the kernel: set it
    // once per device (thread-safe)
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static hipError_t set_rc[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] {
        set_rc[dev] = hipFuncSetAttribute(
            (const void *)gemm_bf16_kernel<BM, BN, BK, STAGES, WGM, WGN, FW, U2>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    });
    if (set_rc[dev] != hipSuccess) return set_rc[dev];
    const int64_t blocks = a.n_blocks;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, STAGES, WGM, WGN, FW, U2>),
                       dim3((unsigned)blocks), dim3(64 * WGM * WGN), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

bool fused_reduce_supported(int32_t bm, int32_t bn, int32_t W) {
    return bm == 256 && bn == 256 && W == 8;
}

bool bf16_tile_supported(int32_t bm, int32_t bn) {
    return (bm == 256 && bn == 256) || (bm == 256 && bn == 128) ||
           (bm == 128 && bn == 128) || (bm == 64 && bn == 128);
}

hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s) {
    const int bm = a.g.BM, bn = a.g.BN;
    // 64-deep K steps in two LDS stages of (BM + BN) x 64 bf16
    constexpr int BKc = 64, ST = 2;
    if (a.fuse_reduce) {
        // the owner-fused reduce exists for W = 8 with 256 x 256 tiles
        if (bm == 256 && bn == 256 && a.g.W == 8)
            return launch_tile<256, 256, BKc, ST, 2, 4, 8>(a, s);
        return hipErrorInvalidValue;
    }
    if (bm == 256 && bn == 256) {
        // the unrolled loop unless this launch shares the CUs with another
        // kernel's waves (all-gather copies: signals; reduce slices: coresident)
        if (!a.signals && !a.coresident) return launch_tile<256, 256, BKc, ST, 2, 4, 0, true>(a, s);
        return launch_tile<256, 256, BKc, ST, 2, 4>(a, s);
    }
    if (bm == 256 && bn == 128) return launch_tile<256, 128, BKc, ST, 2, 2>(a, s);
    if (bm == 128 && bn == 128) return launch_tile<128, 128, BKc, ST, 2, 2>(a, s);
    // 64 x 128 (the m <= 64 decode shard, HBM-bound): four waves of 64 x 32
    // keep more loads in flight per CU than two of 64 x 64 (+2%)
    if (bm == 64 && bn == 128) return launch_tile<64, 128, BKc, ST, 1, 4>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace gemm_rs
