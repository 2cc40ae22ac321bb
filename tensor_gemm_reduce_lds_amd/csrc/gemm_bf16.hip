// bf16 GEMM + reduce-scatter epilogue for gfx950.
//
// Workgroup b computes one BM x BN output tile of rank r = b % W (tile
// order: tile_of_block).  Mainloop: 64-deep K steps, A and B tiles staged
// through LDS (double buffered, 16-byte global loads, XOR-swizzled rows),
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Epilogue: alpha*acc,
// plus beta*C on rows whose chunk this rank owns, stored as fp32 into the
// staging slot of the row's destination chunk; then the tile's ready flag
// is released at agent scope (page "flux实现：sm80 gemm+rs", section
// "cutlass自定义epilogue–sm80": compute node alpha*acc + beta*C, store node
// that scatters by destination, and a per-tile flag).
#include "gemm_rs_internal.h"

namespace gemm_rs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BK = 64;          // K depth of one LDS stage (elements)
constexpr int ROW_ELEMS = BK;   // LDS row: 64 bf16 = 128 bytes = 8 chunks

// 16-byte chunk c of LDS row `row` is stored at chunk swz(row, c).  Rows
// r and r + 8k map their chunks differently, which keeps both the 8x8 B
// transposes and the MFMA operand reads spread over the banks.
__device__ __forceinline__ int swz(int row, int c) {
    return c ^ ((row ^ (row >> 3)) & 7);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int WM = BM / 2, WN = BN / 2;       // 2 x 2 waves
    constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 MFMA blocks per wave
    constexpr int A_LOADS = BM / 32;              // 16-byte A loads per thread
    constexpr int NB = BN / 8;                    // 8-column groups of B
    constexpr int KR = BK * BN / 8 / kThreads;    // B k-rows per thread
    static_assert(KR == 2 || KR == 4 || KR == 8, "B tile split");
    constexpr int STAGE = (BM + BN) * ROW_ELEMS;  // bf16 elements per stage

    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

    const TileGeom &g = a.g;
    int32_t r, t;
    tile_of_block(g, blockIdx.x, &r, &t);
    const int32_t tm = t / g.tiles_n, tn = t - (t / g.tiles_n) * g.tiles_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const uint16_t *A = (const uint16_t *)a.A + (int64_t)r * g.M * g.K;
    const uint16_t *B = (const uint16_t *)a.B + (int64_t)r * g.K * g.N;
    const int64_t row0 = (int64_t)tm * BM;
    const int64_t col0 = (int64_t)tn * BN;

    // per-thread global source pointers (k offset added per stage)
    const uint16_t *a_src[A_LOADS];
#pragma unroll
    for (int p = 0; p < A_LOADS; ++p) {
        int64_t row = row0 + p * 32 + (tid >> 3);
        if (row > g.M - 1) row = g.M - 1;   // ragged M: read a valid row
        a_src[p] = A + row * g.K + (tid & 7) * 8;
    }
    const int nb = tid % NB, kb = tid / NB;
    const uint16_t *b_src = B + (int64_t)(kb * KR) * g.N + col0 + nb * 8;

    u32x4_t a_reg[A_LOADS];
    u32x4_t b_reg[KR];

    auto load_global = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p)
            a_reg[p] = *(const u32x4_t *)(a_src[p] + k0);
#pragma unroll
        for (int e = 0; e < KR; ++e)
            b_reg[e] = *(const u32x4_t *)(b_src + (k0 + e) * g.N);
    };

    auto store_lds = [&](int buf) {
        uint16_t *As = lds + buf * STAGE;
        uint16_t *Bs = As + BM * ROW_ELEMS;
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            const int row = p * 32 + (tid >> 3);
            *(u32x4_t *)(As + row * ROW_ELEMS + swz(row, tid & 7) * 8) = a_reg[p];
        }
        // 8x8 (KR x 8) transpose: B[k][n] -> Bs[n][k] (k contiguous)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int n = nb * 8 + q;
            const int w = q >> 1, sh = (q & 1) * 16;
            uint32_t v[KR];
#pragma unroll
            for (int e = 0; e < KR; ++e) v[e] = (b_reg[e][w] >> sh) & 0xffffu;
            const int kofs = kb * KR;              // element offset in the row
            uint16_t *dst = Bs + n * ROW_ELEMS + swz(n, kofs >> 3) * 8 + (kofs & 7);
            if constexpr (KR == 8) {
                u32x4_t o = {v[0] | (v[1] << 16), v[2] | (v[3] << 16),
                             v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
                *(u32x4_t *)dst = o;
            } else if constexpr (KR == 4) {
                u32x2_t o = {v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
                *(u32x2_t *)dst = o;
            } else {
                *(uint32_t *)dst = v[0] | (v[1] << 16);
            }
        }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto compute = [&](int buf) {
        const uint16_t *As = lds + buf * STAGE;
        const uint16_t *Bs = As + BM * ROW_ELEMS;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = ks * 2 + (lane >> 5);
            bf16x8_t af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WM + i * 32 + (lane & 31);
                af[i] = *(const bf16x8_t *)(As + row * ROW_ELEMS + swz(row, c) * 8);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = wn * WN + j * 32 + (lane & 31);
                bfr[j] = *(const bf16x8_t *)(Bs + n * ROW_ELEMS + swz(n, c) * 8);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    const int KT = (int)(g.K / BK);
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_global(kt + 1);
        compute(cur);
        if (kt + 1 < KT) store_lds(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: D = alpha*acc (+ beta*C on owned rows), scatter ----
    // 32x32 accumulator layout: lane holds column (lane & 31); register v
    // holds row 8*(v/4) + 4*(lane/32) + (v%4) of the 32x32 block.
    const uint16_t *Cp = (const uint16_t *)a.C;
    const float alpha = a.alpha, beta = a.beta;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = row0 + wm * WM + i * 32 + 8 * (v >> 2) +
                                4 * (lane >> 5) + (v & 3);
            if (row >= g.M) continue;
            const int32_t d = (int32_t)((uint32_t)row / (uint32_t)g.Mc);
            const bool own_c = a.has_c && d == r;
            float *dst = a.staging +
                         (((int64_t)d * g.W + r) * g.Mc + (row - (int64_t)d * g.Mc)) * g.N;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t col = col0 + wn * WN + j * 32 + (lane & 31);
                float x = alpha * acc[i][j][v];
                if (own_c) x += beta * bf16_bits_to_float(Cp[row * a.ldc + col]);
                __builtin_nontemporal_store(x, dst + col);
            }
        }
    }

    // ---- publish: all stores of this tile, then flag[r][t] = 1 ----
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        __hip_atomic_store(&a.flags[(int64_t)r * g.T + t], 1u, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (a.trace) a.trace[blockIdx.x] = t;
    }
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs &a, hipStream_t s) {
    constexpr size_t lds_bytes = 2 * (BM + BN) * BK * sizeof(uint16_t);
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(
            (const void *)gemm_bf16_kernel<BM, BN>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const int64_t blocks = (int64_t)a.g.W * a.g.T;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN>), dim3((unsigned)blocks),
                       dim3(kThreads), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

bool bf16_tile_supported(int32_t bm, int32_t bn) {
    return (bm == 256 && bn == 256) || (bm == 256 && bn == 128) ||
           (bm == 128 && bn == 128) || (bm == 64 && bn == 128);
}

hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s) {
    const int bm = a.g.BM, bn = a.g.BN;
    if (bm == 256 && bn == 256) return launch_tile<256, 256>(a, s);
    if (bm == 256 && bn == 128) return launch_tile<256, 128>(a, s);
    if (bm == 128 && bn == 128) return launch_tile<128, 128>(a, s);
    if (bm == 64 && bn == 128) return launch_tile<64, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace gemm_rs
