/*
 * oracle_w4a8.c -- plain, slow CPU oracle for block-scaled int8 activation
 * quantization and the W4A8 grouped GEMM that consumes it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and never calls it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * With those flags on x86-64 (SSE2, FLT_EVAL_METHOD == 0) every float
 * expression below is a sequence of single IEEE-754 binary32 operations with
 * round-to-nearest-even, in source order: no fused multiply-add, no
 * re-association, no flush-to-zero.  OpenMP only splits independent outputs
 * (rows / output channels), so results do not depend on the thread count.
 *
 * Pages this follows (cited by page title and section):
 *   [EQuARX]   "EQuARX" verdict page, pith.science arXiv 2506.17615:
 *              pith_extraction.key_machinery -- symmetric block-wise int8,
 *              absmax per block, one FP32 scale per block, quantization in two
 *              phases (Qp1 computes the scales, Qp2 scales the data), and
 *              dequantization back to FP32.
 *   [LiquidGEMM] "LiquidGEMM" verdict page, pith.science arXiv 2509.01229:
 *              referee_report.summary and skeptic_critique.load_bearing_attack
 *              -- two-level weight quantization: an INT8 first level, then a
 *              4-bit second level with an integer per-group scale;
 *              referee_report.major_comments[2] (paper section 4, Eq. 7) --
 *              protective range of the INT8 level and integer group scale
 *              bounded by 16; pith_extraction.key_machinery -- the
 *              (u4 * s + a) XOR 0x80 dequantization identity.
 *   [HBQ]      "HBQ: Hierarchical Scaling Block Quantization" episode page,
 *              section "Improvements" -- hierarchical (two-level) scaling.
 *
 * Readings taken where the pages leave a step open (each is also listed in
 * the design notes):
 *   R1  Activation codes are symmetric int8 in [-127, 127]; scale = amax/127.
 *   R2  The code is rne(x * fl(127/amax)): one binary32 multiply by the
 *       rounded reciprocal, then round-half-even to an integer.
 *   R3  amax == 0 gives scale 0, inverse 0 and all codes 0.  If 127/amax
 *       overflows (amax below about 2^-121) the inverse is +inf; the code
 *       conversion saturates at the range ends and maps NaN (0 * inf) to 0.
 *   R4  Weights: per-channel level 1 with protective range 112 (= 7 * 16) so
 *       the integer group scale stays in [1, 16]; level 2 per group of 64:
 *       s_g = max(1, ceil(m_g / 7)), q = exact-rational round-half-even of
 *       W8 / s_g, codes in [-7, 7].
 *   R5  GEMM: per-token activation scales; acc = sum_g s_g * P_g in int32
 *       where P_g is the int32 dot product over group g; the real output is
 *       acc * s_a[m] * s_ch[n], computed here in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)

/* Largest K for which |acc| <= K * 127 * 112 still fits in int32. */
#define ORACLE_K_MAX 150976

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 -> binary32 is exact: the bf16 bits are the high half of the float. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/* Round v half-to-even and saturate to [-lim, lim]; NaN gives 0 (R3). */
static int saturating_round_half_even(float v, int lim)
{
    if (v != v)
        return 0;
    if (v >= (float)lim)
        return lim;
    if (v <= -(float)lim)
        return -lim;
    /* rintf follows the current rounding mode, which is round-to-nearest-even */
    return (int)rintf(v);
}

/* --------------------------------------------- activations: Qp1 + Qp2 -- */

/*
 * Block-wise symmetric int8 quantization of a bf16 [rows, cols] tensor.
 * Blocks are `block` contiguous elements along a row ([EQuARX]
 * pith_extraction.key_machinery: one FP32 scale per block, absmax reduction,
 * then scaling of the data).  Outputs: q [rows, cols] int8 and
 * scales [rows, cols/block] binary32.
 */
int oracle_quantize_act_blockwise(const uint16_t *x, int64_t rows, int64_t cols,
                                  int32_t block, int8_t *q, float *scales)
{
    if (rows < 0 || cols < 0 || block <= 0 || (cols % block) != 0)
        return ORACLE_BAD_ARGS;
    if (rows == 0 || cols == 0)
        return ORACLE_OK;
    if (!x || !q || !scales)
        return ORACLE_BAD_ARGS;
    const int64_t nblk = cols / block;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            const uint16_t *xb = x + r * cols + b * block;
            int8_t *qb = q + r * cols + b * block;
            /* Qp1: absmax of the block (exact), scale and its inverse. */
            float amax = 0.0f;
            for (int32_t i = 0; i < block; ++i) {
                float a = fabsf(bf16_bits_to_float(xb[i]));
                if (a > amax)
                    amax = a;
            }
            float s = amax / 127.0f;
            float inv = (amax > 0.0f) ? (127.0f / amax) : 0.0f;
            scales[r * nblk + b] = s;
            /* Qp2: scale every element and round to the int8 code. */
            for (int32_t i = 0; i < block; ++i) {
                float v = bf16_bits_to_float(xb[i]) * inv;
                qb[i] = (int8_t)saturating_round_half_even(v, 127);
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Dequantization back to binary32 ([EQuARX] pith_extraction.key_machinery:
 * received blocks are dequantized to FP32): x_hat = q * s, one binary32
 * multiply.  out_f32 and/or out_bf16 (bf16 = RNE of the binary32 value) may
 * be NULL.
 */
int oracle_dequantize_act_blockwise(const int8_t *q, const float *scales, int64_t rows,
                                    int64_t cols, int32_t block, float *out_f32,
                                    uint16_t *out_bf16)
{
    if (rows < 0 || cols < 0 || block <= 0 || (cols % block) != 0)
        return ORACLE_BAD_ARGS;
    if (rows == 0 || cols == 0)
        return ORACLE_OK;
    if (!q || !scales)
        return ORACLE_BAD_ARGS;
    const int64_t nblk = cols / block;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            float v = (float)q[r * cols + c] * scales[r * nblk + c / block];
            if (out_f32)
                out_f32[r * cols + c] = v;
            if (out_bf16)
                out_bf16[r * cols + c] = float_to_bf16_bits(v);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------ weights: two levels -- */

/*
 * Level 1 (per output channel n): c = max_k |w[n,k]|, s_ch = c / 112,
 * W8 = clamp(rne(w * fl(112 / c)), -112, 112).  The INT8 first level and its
 * protective range follow [LiquidGEMM] referee_report.summary and
 * referee_report.major_comments[2]; the range 112 is reading R4.
 */
int oracle_weight_level1(const uint16_t *w, int64_t n, int64_t k, int8_t *w8, float *s_ch)
{
    if (n < 0 || k < 0)
        return ORACLE_BAD_ARGS;
    if (n == 0 || k == 0)
        return ORACLE_OK;
    if (!w || !w8 || !s_ch)
        return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t *wr = w + r * k;
        float c = 0.0f;
        for (int64_t i = 0; i < k; ++i) {
            float a = fabsf(bf16_bits_to_float(wr[i]));
            if (a > c)
                c = a;
        }
        s_ch[r] = c / 112.0f;
        float inv = (c > 0.0f) ? (112.0f / c) : 0.0f;
        for (int64_t i = 0; i < k; ++i) {
            float v = bf16_bits_to_float(wr[i]) * inv;
            w8[r * k + i] = (int8_t)saturating_round_half_even(v, 112);
        }
    }
    return ORACLE_OK;
}

/* Exact rational a / s rounded half to even, for integers a and s >= 1. */
static int div_round_half_even(int a, int s)
{
    int neg = a < 0;
    int m = neg ? -a : a;
    int quo = m / s;
    int rem = m % s;
    if (2 * rem > s || (2 * rem == s && (quo & 1)))
        quo += 1;
    return neg ? -quo : quo;
}

/*
 * Level 2 (per channel n and group g of `group` consecutive k): m_g =
 * max |W8|, integer scale s_g = max(1, ceil(m_g / 7)) in [1, 16], code
 * q = rne(W8 / s_g) in [-7, 7] ([LiquidGEMM] skeptic_critique.
 * load_bearing_attack: the group scale is rounded to an integer;
 * referee_report.major_comments[2]: it is at most 16; reading R4 fixes the
 * rounding of the scale to ceil so no code is clamped).
 * Outputs: q [n, k] int8 and s_g [n, k/group] uint8 in plain row-major order.
 */
int oracle_weight_level2(const int8_t *w8, int64_t n, int64_t k, int32_t group, int8_t *q,
                         uint8_t *s_g)
{
    if (n < 0 || k < 0 || group <= 0 || (k % group) != 0)
        return ORACLE_BAD_ARGS;
    if (n == 0 || k == 0)
        return ORACLE_OK;
    if (!w8 || !q || !s_g)
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const int8_t *src = w8 + r * k + g * group;
            int m = 0;
            for (int32_t i = 0; i < group; ++i) {
                int a = src[i] < 0 ? -src[i] : src[i];
                if (a > m)
                    m = a;
            }
            int s = (m == 0) ? 1 : (m + 6) / 7;
            s_g[r * ng + g] = (uint8_t)s;
            for (int32_t i = 0; i < group; ++i) {
                int v = div_round_half_even(src[i], s);
                if (v > 7)
                    v = 7;
                if (v < -7)
                    v = -7;
                q[r * k + g * group + i] = (int8_t)v;
            }
        }
    }
    return ORACLE_OK;
}

/* Both weight levels: bf16 w [n, k] -> canonical q, s_g, s_ch. */
int oracle_quantize_w4_grouped(const uint16_t *w, int64_t n, int64_t k, int32_t group,
                               int8_t *q, uint8_t *s_g, float *s_ch)
{
    if (n < 0 || k < 0 || group <= 0 || (k % group) != 0)
        return ORACLE_BAD_ARGS;
    if (n == 0 || k == 0)
        return ORACLE_OK;
    int8_t *w8 = (int8_t *)malloc((size_t)(n * k));
    if (!w8)
        return ORACLE_BAD_ARGS;
    int rc = oracle_weight_level1(w, n, k, w8, s_ch);
    if (rc == ORACLE_OK)
        rc = oracle_weight_level2(w8, n, k, group, q, s_g);
    free(w8);
    return rc;
}

/* Effective weight w_hat[n,k] = s_ch[n] * (s_g[n,g] * q[n,k]) in binary64. */
int oracle_dequantize_w4_grouped(const int8_t *q, const uint8_t *s_g, const float *s_ch,
                                 int64_t n, int64_t k, int32_t group, double *w_hat)
{
    if (n < 0 || k < 0 || group <= 0 || (k % group) != 0)
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < k; ++i)
            w_hat[r * k + i] =
                (double)s_ch[r] * (double)(s_g[r * ng + i / group] * q[r * k + i]);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- GEMM -- */

/*
 * Per-group int32 dot products P[m, n, g] = sum_{k in group g} a_q[m,k] * q[n,k]
 * (int8 x int8 products accumulated in int32).
 */
int oracle_group_sums(const int8_t *a_q, const int8_t *q, int64_t m, int64_t n, int64_t k,
                      int32_t group, int32_t *P)
{
    if (m < 0 || n < 0 || k < 0 || group <= 0 || (k % group) != 0)
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            for (int64_t g = 0; g < ng; ++g) {
                int32_t sum = 0;
                for (int32_t t = 0; t < group; ++t)
                    sum += (int32_t)a_q[i * k + g * group + t] *
                           (int32_t)q[j * k + g * group + t];
                P[(i * n + j) * ng + g] = sum;
            }
    return ORACLE_OK;
}

/*
 * W4A8 GEMM on canonical operands.
 *   acc[m,n] = sum_g s_g[n,g] * P[m,n,g]       (int32, exact; group scales
 *                                               applied per K-group)
 *   y[m,n]   = acc[m,n] * s_a[m] * s_ch[n]      (binary64; may be NULL)
 * a_q [m,k] int8, a_scale [m] (per-token scale), q [n,k] int8 in [-7,7],
 * s_g [n,k/group] uint8, s_ch [n] binary32.
 */
int oracle_w4a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *q,
                     const uint8_t *s_g, const float *s_ch, int64_t m, int64_t n, int64_t k,
                     int32_t group, int32_t *acc, double *y)
{
    if (m < 0 || n < 0 || k < 0 || group <= 0 || (k % group) != 0 || k > ORACLE_K_MAX)
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int32_t total = 0;
            for (int64_t g = 0; g < ng; ++g) {
                int32_t p = 0;
                for (int32_t t = 0; t < group; ++t)
                    p += (int32_t)a_q[i * k + g * group + t] *
                         (int32_t)q[j * k + g * group + t];
                total += (int32_t)s_g[j * ng + g] * p;
            }
            if (acc)
                acc[i * n + j] = total;
            if (y)
                y[i * n + j] = (double)total * (double)a_scale[i] * (double)s_ch[j];
        }
    }
    return ORACLE_OK;
}

/*
 * Fused form: per-token quantization of bf16 activations (block = k) followed
 * by the GEMM.  a_q_out [m,k] and a_s_out [m] receive the activation codes
 * and scales.
 */
int oracle_w4a8_gemm_bf16act(const uint16_t *a, const int8_t *q, const uint8_t *s_g,
                             const float *s_ch, int64_t m, int64_t n, int64_t k,
                             int32_t group, int8_t *a_q_out, float *a_s_out, int32_t *acc,
                             double *y)
{
    if (k <= 0)
        return ORACLE_BAD_ARGS;
    int rc = oracle_quantize_act_blockwise(a, m, k, (int32_t)k, a_q_out, a_s_out);
    if (rc != ORACLE_OK)
        return rc;
    return oracle_w4a8_gemm(a_q_out, a_s_out, q, s_g, s_ch, m, n, k, group, acc, y);
}

/* Number of threads the OpenMP regions above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
