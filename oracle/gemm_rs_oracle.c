/*
 * CPU oracle for the fused GEMM + reduce-scatter path.  TEST INFRASTRUCTURE
 * ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg call
 * it; the product path never does.  It shares no code with the HIP library.
 *
 * What it computes, from the pages:
 *   - Each of W ranks multiplies its own A_r[M,K] by B_r[K,N]; the GEMM's
 *     epilogue computes alpha*acc + beta*C and writes the tile into the
 *     reduce-scatter buffer instead of an ordinary output (page
 *     "flux实现：sm80 gemm+rs", opening paragraph and section
 *     "cutlass自定义epilogue–sm80", nodes EVT_Compute0 / EVT_Compute1).
 *   - Rank d of the reduce-scatter receives rows [d*M/W, (d+1)*M/W) of the
 *     sum over ranks (page "flux精读", section 3 Design; page
 *     "通信 overlap 实现", section on Flux tile fusion, GEMM+RS bullet).
 *   - The sum is either flat or two-level: partial sums within each group of
 *     ranks first, then across groups (page "flux实现：sm80 gemm+rs",
 *     section "2D Ring优化").
 *
 * Readings taken where the pages are silent:
 *   - beta*C is a bias that must appear once in the result, so it is added
 *     only in the partial of the rank that owns the row's chunk (r == d(i)).
 *   - the flat order is ascending r; the two-level order uses contiguous
 *     groups of W/G ranks, ascending inside each group, then ascending over
 *     groups.
 *   - ldc == 0 means C is one row broadcast down all rows.
 *
 * Two numeric modes:
 *   reference : everything in double, no rounding (the parity target).
 *   emulate   : each rank's epilogue value rounded to float, the ordered sum
 *               done in float, the result rounded to bfloat16 by
 *               round-to-nearest-even (or kept as float).  It reproduces a
 *               float pipeline bit for bit only where every epilogue value is
 *               exact in float (small-integer inputs).
 *
 * dtype 0: bfloat16 inputs given as uint16 bit patterns; dtype 1: float32.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_F32 = 1 };
enum { OR_FLAT = 0, OR_TWO_LEVEL = 1 };
enum { OUT_BF16 = 0, OUT_F32 = 1 };

/* bfloat16 bits -> double: the bits are the top half of a float. */
static double bf16_bits_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int32_t dtype, int64_t idx)
{
    if (dtype == OR_BF16)
        return bf16_bits_value(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/*
 * float -> bfloat16 bits, round to nearest, ties to even.  bfloat16 keeps
 * the top 16 bits of the float; the dropped low half decides the rounding.
 * NaN stays NaN (quiet bit set); infinities and overflow to infinity follow
 * from the integer carry.
 */
uint16_t oracle_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

void oracle_bf16_rne_array(int64_t n, const float *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(x[i]);
}

/* Threads the next parallel region may use (timing a single-thread baseline). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Epilogue value of rank r for row i, all N columns, in double:
 *   D_r[i][j] = alpha * sum_k A_r[i][k] * B_r[k][j]
 *               + (r == d(i) and has_c ? beta * C[i][j] : 0)
 * The k sum runs in ascending k for every j.
 */
static void rank_row(int64_t M, int64_t N, int64_t K, int32_t W, int32_t dtype,
                     const void *A, const void *B, const void *C,
                     int32_t has_c, int64_t ldc, double alpha, double beta,
                     int32_t r, int64_t i, double *row)
{
    int64_t Mc = M / W;
    int64_t d = i / Mc;
    for (int64_t j = 0; j < N; ++j)
        row[j] = 0.0;
    const int64_t a_off = ((int64_t)r * M + i) * K;
    const int64_t b_off = (int64_t)r * K * N;
    for (int64_t k = 0; k < K; ++k) {
        double a = load_elem(A, dtype, a_off + k);
        const int64_t brow = b_off + k * N;
        for (int64_t j = 0; j < N; ++j)
            row[j] += a * load_elem(B, dtype, brow + j);
    }
    for (int64_t j = 0; j < N; ++j)
        row[j] *= alpha;
    if (has_c && (int64_t)r == d) {
        const int64_t c_off = i * ldc; /* ldc == 0: the same row for every i */
        for (int64_t j = 0; j < N; ++j)
            row[j] += beta * load_elem(C, dtype, c_off + j);
    }
}

static int check_shape(int64_t M, int64_t N, int64_t K, int32_t W,
                       int32_t order, int32_t groups)
{
    /* K == 0 is the empty sum: every partial is 0 */
    if (M <= 0 || N <= 0 || K < 0 || W <= 0 || M % W != 0)
        return -1;
    if (order == OR_TWO_LEVEL && (groups <= 0 || W % groups != 0))
        return -1;
    if (order != OR_FLAT && order != OR_TWO_LEVEL)
        return -1;
    return 0;
}

/* Epilogue values of one rank for rows [row_lo, row_hi), in double. */
int oracle_partial_rows(int64_t M, int64_t N, int64_t K, int32_t W,
                        int32_t dtype, const void *A, const void *B,
                        const void *C, int32_t has_c, int64_t ldc,
                        double alpha, double beta, int32_t r,
                        int64_t row_lo, int64_t row_hi, double *out)
{
    if (check_shape(M, N, K, W, OR_FLAT, 1) || r < 0 || r >= W ||
        row_lo < 0 || row_hi > M || row_lo > row_hi)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_lo; i < row_hi; ++i)
        rank_row(M, N, K, W, dtype, A, B, C, has_c, ldc, alpha, beta, r, i,
                 out + (i - row_lo) * N);
    return 0;
}

/*
 * Reference mode, rows [row_lo, row_hi) of the reduced result, in double.
 * Flat: y = ((D_0 + D_1) + ...) + D_{W-1}.
 * Two-level: S_g = ascending sum over the L = W/G ranks of group g
 * (ranks g*L .. g*L+L-1), then y = ((S_0 + S_1) + ...) + S_{G-1}.
 */
int oracle_reference_rows(int64_t M, int64_t N, int64_t K, int32_t W,
                          int32_t dtype, const void *A, const void *B,
                          const void *C, int32_t has_c, int64_t ldc,
                          double alpha, double beta, int32_t order,
                          int32_t groups, int64_t row_lo, int64_t row_hi,
                          double *out)
{
    if (check_shape(M, N, K, W, order, groups) || row_lo < 0 ||
        row_hi > M || row_lo > row_hi)
        return -1;
    int32_t L = (order == OR_TWO_LEVEL) ? W / groups : W;
    int fail = 0;
#pragma omp parallel
    {
        double *d_r = (double *)malloc(sizeof(double) * (size_t)N);
        double *s_g = (double *)malloc(sizeof(double) * (size_t)N);
        if (!d_r || !s_g) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row_lo; i < row_hi; ++i) {
                double *y = out + (i - row_lo) * N;
                for (int32_t r = 0; r < W; ++r) {
                    rank_row(M, N, K, W, dtype, A, B, C, has_c, ldc, alpha,
                             beta, r, i, d_r);
                    int first_in_group = (r % L) == 0;
                    for (int64_t j = 0; j < N; ++j)
                        s_g[j] = first_in_group ? d_r[j] : s_g[j] + d_r[j];
                    if ((r % L) == L - 1) {
                        int first_group = (r / L) == 0;
                        for (int64_t j = 0; j < N; ++j)
                            y[j] = first_group ? s_g[j] : y[j] + s_g[j];
                    }
                }
            }
        }
        free(d_r);
        free(s_g);
    }
    return fail ? -2 : 0;
}

/*
 * Emulate mode, rows [row_lo, row_hi): D_r rounded to float (and, with
 * staging_kind 1, that float rounded to bfloat16 by RNE, the value a
 * bfloat16 staging slot holds), the ordered sum (same order as reference
 * mode) in float, then bfloat16 RNE bits (out_kind 0, out is uint16) or
 * float (out_kind 1, out is float).
 */
int oracle_emulate_rows(int64_t M, int64_t N, int64_t K, int32_t W,
                        int32_t dtype, const void *A, const void *B,
                        const void *C, int32_t has_c, int64_t ldc,
                        double alpha, double beta, int32_t order,
                        int32_t groups, int64_t row_lo, int64_t row_hi,
                        int32_t out_kind, int32_t staging_kind, void *out)
{
    if (check_shape(M, N, K, W, order, groups) || row_lo < 0 ||
        row_hi > M || row_lo > row_hi)
        return -1;
    int32_t L = (order == OR_TWO_LEVEL) ? W / groups : W;
    int fail = 0;
#pragma omp parallel
    {
        double *d_r = (double *)malloc(sizeof(double) * (size_t)N);
        float *s_g = (float *)malloc(sizeof(float) * (size_t)N);
        float *y = (float *)malloc(sizeof(float) * (size_t)N);
        if (!d_r || !s_g || !y) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row_lo; i < row_hi; ++i) {
                for (int32_t r = 0; r < W; ++r) {
                    rank_row(M, N, K, W, dtype, A, B, C, has_c, ldc, alpha,
                             beta, r, i, d_r);
                    int first_in_group = (r % L) == 0;
                    for (int64_t j = 0; j < N; ++j) {
                        float v = (float)d_r[j];
                        if (staging_kind == 1)
                            v = (float)bf16_bits_value(oracle_bf16_rne(v));
                        s_g[j] = first_in_group ? v : s_g[j] + v;
                    }
                    if ((r % L) == L - 1) {
                        int first_group = (r / L) == 0;
                        for (int64_t j = 0; j < N; ++j)
                            y[j] = first_group ? s_g[j] : y[j] + s_g[j];
                    }
                }
                int64_t base = (i - row_lo) * N;
                if (out_kind == OUT_BF16) {
                    for (int64_t j = 0; j < N; ++j)
                        ((uint16_t *)out)[base + j] = oracle_bf16_rne(y[j]);
                } else {
                    memcpy((float *)out + base, y, sizeof(float) * (size_t)N);
                }
            }
        }
        free(d_r);
        free(s_g);
        free(y);
    }
    return fail ? -2 : 0;
}

/*
 * Reference mode at single elements (i[n], j[n]), in double: one dot
 * product of length K per rank, summed in the same order as above.
 */
int oracle_reference_elems(int64_t M, int64_t N, int64_t K, int32_t W,
                           int32_t dtype, const void *A, const void *B,
                           const void *C, int32_t has_c, int64_t ldc,
                           double alpha, double beta, int32_t order,
                           int32_t groups, int64_t n, const int64_t *ii,
                           const int64_t *jj, double *out)
{
    if (check_shape(M, N, K, W, order, groups))
        return -1;
    for (int64_t e = 0; e < n; ++e)
        if (ii[e] < 0 || ii[e] >= M || jj[e] < 0 || jj[e] >= N)
            return -1;
    int32_t L = (order == OR_TWO_LEVEL) ? W / groups : W;
    int64_t Mc = M / W;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t e = 0; e < n; ++e) {
        int64_t i = ii[e], j = jj[e], d = i / Mc;
        double y = 0.0, s = 0.0;
        for (int32_t r = 0; r < W; ++r) {
            double p = 0.0;
            for (int64_t k = 0; k < K; ++k)
                p += load_elem(A, dtype, ((int64_t)r * M + i) * K + k) *
                     load_elem(B, dtype, ((int64_t)r * K + k) * N + j);
            double v = alpha * p;
            if (has_c && (int64_t)r == d)
                v += beta * load_elem(C, dtype, i * ldc + j);
            s = (r % L == 0) ? v : s + v;
            if (r % L == L - 1)
                y = (r / L == 0) ? s : y + s;
        }
        out[e] = y;
    }
    return 0;
}

/*
 * The ordered float reduction alone, for staging contents written by a
 * test: S is [W][n] floats (slot r of each element at S[r*n + e]).
 */
int oracle_reduce_emulate(int32_t W, int32_t order, int32_t groups, int64_t n,
                          const float *S, int32_t out_kind, void *out)
{
    if (W <= 0 || n < 0)
        return -1;
    if (order == OR_TWO_LEVEL && (groups <= 0 || W % groups != 0))
        return -1;
    if (order != OR_FLAT && order != OR_TWO_LEVEL)
        return -1;
    int32_t L = (order == OR_TWO_LEVEL) ? W / groups : W;
    for (int64_t e = 0; e < n; ++e) {
        float y = 0.0f, s = 0.0f;
        for (int32_t r = 0; r < W; ++r) {
            float v = S[(int64_t)r * n + e];
            s = (r % L == 0) ? v : s + v;
            if (r % L == L - 1)
                y = (r / L == 0) ? s : y + s;
        }
        if (out_kind == OUT_BF16)
            ((uint16_t *)out)[e] = oracle_bf16_rne(y);
        else
            ((float *)out)[e] = y;
    }
    return 0;
}
