// fp32 GEMM + reduce-scatter epilogue for gfx950 (fp32 in, fp32 out).
//
// Same tile order, epilogue and flag protocol as the bf16 kernel, on
// v_mfma_f32_32x32x2_f32: 64x64 tiles, 4 waves of 32x32, 64-deep K steps.
#include "gemm_rs_internal.h"

namespace gemm_rs {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 64, BN = 64, BK = 64;
constexpr int A_PITCH = BK + 1;   // padded rows: column reads hit distinct banks

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs a) {
    __shared__ float As[BM * A_PITCH];
    __shared__ __attribute__((aligned(16))) float Bs[BK * BN];

    const TileGeom &g = a.g;
    int32_t r, t;
    const uint32_t b = a.b_offset + blockIdx.x;
    tile_of_block(g, b, &r, &t);
    const int32_t tm = t / g.tiles_n, tn = t - (t / g.tiles_n) * g.tiles_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const float *A = (const float *)a.A + (int64_t)r * g.M * g.K;
    const float *B = (const float *)a.B + (int64_t)r * g.K * g.N;
    const int64_t row0 = (int64_t)tm * BM, col0 = (int64_t)tn * BN;

    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

    const int KT = (int)(g.K / BK);
    for (int kt = 0; kt < KT; ++kt) {
        const int64_t k0 = (int64_t)kt * BK;
        f32x4_t ar[4], br[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            int64_t row = row0 + p * 16 + (tid >> 4);
            if (row > g.M - 1) row = g.M - 1;
            ar[p] = *(const f32x4_t *)(A + row * g.K + k0 + (tid & 15) * 4);
            br[p] = *(const f32x4_t *)(B + (k0 + p * 16 + (tid >> 4)) * g.N + col0 +
                                       (tid & 15) * 4);
        }
        __syncthreads();   // previous step's reads are done
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = p * 16 + (tid >> 4), kc = (tid & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) As[row * A_PITCH + kc + e] = ar[p][e];
            *(f32x4_t *)(Bs + (p * 16 + (tid >> 4)) * BN + (tid & 15) * 4) = br[p];
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 2; ++ks) {
            const int k = ks * 2 + (lane >> 5);
            const float av = As[(wm * 32 + (lane & 31)) * A_PITCH + k];
            const float bv = Bs[k * BN + wn * 32 + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
        }
    }

    const float *Cp = (const float *)a.C;
    const int64_t col = col0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row >= g.M) continue;
        const int32_t d = (int32_t)((uint32_t)row / (uint32_t)g.Mc);
        float x = a.alpha * acc[v];
        if (a.has_c && d == r) x = __builtin_fmaf(a.beta, Cp[row * a.ldc + col], x);
        float *dst = (float *)a.staging +
                     ((int64_t)d * g.W + r) * g.slot + (row - (int64_t)d * g.Mc) * g.N;
        __builtin_nontemporal_store(x, dst + col);
    }

    // flag publish: the consumer (the reduce) is stream-ordered after this
    // kernel, whose boundary makes the stores visible, so the flag is a
    // plain store
    if (tid == 0) {
        __hip_atomic_store(&a.flags[(int64_t)r * g.T + t], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (a.trace) a.trace[b] = t;
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
    if (a.g.BM != BM || a.g.BN != BN) return hipErrorInvalidValue;
    const int64_t blocks = a.n_blocks;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gemm_rs
