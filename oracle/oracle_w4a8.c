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
 *
 * Readings for the extensions further down (same pages):
 *   R6  LQQ weights (LiquidGEMM's own asymmetric format): level 1 per channel
 *       with protective range 119, Q = clamp(rne(w * fl(119/c)), -119, 119),
 *       s_ch = c/119.  Level 2 per group of 64: min and max of Q; integer
 *       scale s_u8 = max(1, nearest integer to (max - min)/15) -- the page's
 *       bound of 16 on s_u8 holds for rounding to nearest (a tie cannot occur:
 *       15 is odd); code q_u4 = rne((Q - min)/s_u8) clamped to [0, 15]; the
 *       offset stored with the group is min.  The rebuilt int8 operand is
 *       q_u4 * s_u8 + min, in [-119, 127].
 *   R7  Per-block activation scales inside the GEMM (block 32 or a multiple
 *       of 64): the int32 partial of each activation block is exact; the
 *       output is s_ch[n] * sum_b s_a[m,b] * partial_b, here in binary64, with
 *       the bound sum_b |s_a[m,b] * partial_b| * s_ch[n] that fixes the
 *       tolerance of a binary32 fold.
 *   R8  W8A8 comparison path: symmetric int8 weights per channel (range
 *       127), per-token int8 activations, exact int32 accumulation.
 *   R9  EQuARX local reduction step: a received int8 block is dequantized to
 *       binary32 (q * s), added in binary32 to the local partial sum (binary32,
 *       or bf16 widened exactly), and the sum is requantized with R1-R3.
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

/* ------------------------------------------- extension: LQQ weights -- */

/* Largest K with |acc| <= K * 127 * 127 in int32, rounded down to a multiple
 * of 64 (LQQ operands reach 127; so do W8A8 weights). */
#define ORACLE_K_MAX_127 133120

/* Per-channel symmetric int8 level with protective range `range`:
 * c = max |w|, s_ch = c / range, code = clamp(rne(w * fl(range / c))). */
static void channel_int8(const uint16_t *w, int64_t n, int64_t k, int range, int8_t *w8,
                         float *s_ch)
{
    const float fr = (float)range;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t *wr = w + r * k;
        float c = 0.0f;
        for (int64_t i = 0; i < k; ++i) {
            float a = fabsf(bf16_bits_to_float(wr[i]));
            if (a > c)
                c = a;
        }
        s_ch[r] = c / fr;
        float inv = (c > 0.0f) ? (fr / c) : 0.0f;
        for (int64_t i = 0; i < k; ++i)
            w8[r * k + i] = (int8_t)saturating_round_half_even(bf16_bits_to_float(wr[i]) * inv,
                                                               range);
    }
}

/*
 * LQQ ("LiquidGEMM" verdict page, pith_extraction.key_machinery: the int8
 * weights are shifted by the group minimum into the unsigned domain, coded on
 * 4 bits with an integer scale, and rebuilt as (q_u4 * s_u8 + a) XOR 0x80 with
 * a = 128 + min; referee_report.major_comments[2]: protective range 119 and
 * s_u8 <= 16).  Reading R6.  Outputs in plain row-major order:
 * q_u4 [n,k] in [0,15], s_u8 [n,k/group] in [1,16], w_min [n,k/group] in
 * [-119,119], s_ch [n].
 */
int oracle_quantize_w4_lqq(const uint16_t *w, int64_t n, int64_t k, int32_t group,
                           uint8_t *q_u4, uint8_t *s_u8, int8_t *w_min, float *s_ch)
{
    if (n < 0 || k < 0 || group <= 0 || (k % group) != 0)
        return ORACLE_BAD_ARGS;
    if (n == 0)
        return ORACLE_OK;
    if (!w || !s_ch)
        return ORACLE_BAD_ARGS;
    if (k == 0) {
        for (int64_t r = 0; r < n; ++r)
            s_ch[r] = 0.0f;
        return ORACLE_OK;
    }
    if (!q_u4 || !s_u8 || !w_min)
        return ORACLE_BAD_ARGS;
    int8_t *w8 = (int8_t *)malloc((size_t)(n * k));
    if (!w8)
        return ORACLE_BAD_ARGS;
    channel_int8(w, n, k, 119, w8, s_ch);
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const int8_t *src = w8 + r * k + g * group;
            int lo = src[0], hi = src[0];
            for (int32_t i = 1; i < group; ++i) {
                if (src[i] < lo)
                    lo = src[i];
                if (src[i] > hi)
                    hi = src[i];
            }
            /* nearest integer to (hi - lo) / 15; 15 is odd, so never a tie */
            int span = hi - lo;
            int s = span / 15 + ((span % 15) * 2 > 15 ? 1 : 0);
            if (s < 1)
                s = 1;
            s_u8[r * ng + g] = (uint8_t)s;
            w_min[r * ng + g] = (int8_t)lo;
            for (int32_t i = 0; i < group; ++i) {
                int v = div_round_half_even(src[i] - lo, s);
                if (v > 15)
                    v = 15;
                q_u4[r * k + g * group + i] = (uint8_t)v;
            }
        }
    }
    free(w8);
    return ORACLE_OK;
}

/* Effective LQQ weight s_ch[n] * (q_u4 * s_u8 + min) in binary64. */
int oracle_dequantize_w4_lqq(const uint8_t *q_u4, const uint8_t *s_u8, const int8_t *w_min,
                             const float *s_ch, int64_t n, int64_t k, int32_t group,
                             double *w_hat)
{
    if (n < 0 || k < 0 || group <= 0 || (k % group) != 0)
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < k; ++i) {
            int g = (int)(i / group);
            int op = (int)q_u4[r * k + i] * (int)s_u8[r * ng + g] + (int)w_min[r * ng + g];
            w_hat[r * k + i] = (double)s_ch[r] * (double)op;
        }
    return ORACLE_OK;
}

/*
 * W4A8 GEMM on LQQ weights: acc[m,n] = sum_k a_q[m,k] * (q_u4 * s_u8 + min)
 * in int32 (exact: |acc| <= K * 127 * 127), y = acc * s_a[m] * s_ch[n] in
 * binary64 (may be NULL).
 */
int oracle_w4a8_gemm_lqq(const int8_t *a_q, const float *a_scale, const uint8_t *q_u4,
                         const uint8_t *s_u8, const int8_t *w_min, const float *s_ch,
                         int64_t m, int64_t n, int64_t k, int32_t group, int32_t *acc,
                         double *y)
{
    if (m < 0 || n < 0 || k < 0 || group <= 0 || (k % group) != 0 || k > ORACLE_K_MAX_127)
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int32_t total = 0;
            for (int64_t t = 0; t < k; ++t) {
                int64_t g = t / group;
                int32_t op = (int32_t)q_u4[j * k + t] * (int32_t)s_u8[j * ng + g] +
                             (int32_t)w_min[j * ng + g];
                total += (int32_t)a_q[i * k + t] * op;
            }
            if (acc)
                acc[i * n + j] = total;
            if (y)
                y[i * n + j] = (double)total * (double)a_scale[i] * (double)s_ch[j];
        }
    }
    return ORACLE_OK;
}

/* ------------------- extension: per-block activation scales in the GEMM -- */

/*
 * Reading R7.  a_scale is [m, k/block] (the block quantizer's scales);
 * block is 32 or a multiple of the weight group 64, and divides k.
 *   partial_b[m,n] = sum_{k in block b} a_q[m,k] * q[n,k] * s_g[n, k/group]  (int32)
 *   y[m,n]     = s_ch[n] * sum_b s_a[m,b] * partial_b                       (binary64)
 *   bound[m,n] = s_ch[n] * sum_b |s_a[m,b] * partial_b|                     (binary64)
 * bound (may be NULL) scales the error of any binary32 evaluation of the sum.
 */
int oracle_w4a8_gemm_blockact(const int8_t *a_q, const float *a_scale, const int8_t *q,
                              const uint8_t *s_g, const float *s_ch, int64_t m, int64_t n,
                              int64_t k, int32_t group, int32_t block, double *y,
                              double *bound)
{
    if (m < 0 || n < 0 || k < 0 || group <= 0 || (k % group) != 0 || k > ORACLE_K_MAX ||
        block <= 0 || (k % block) != 0 || !(group % block == 0 || block % group == 0))
        return ORACLE_BAD_ARGS;
    const int64_t ng = k / group, nb = k / block;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double sum = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t part = 0;
                for (int64_t t = b * block; t < (b + 1) * block; ++t)
                    part += (int32_t)a_q[i * k + t] * (int32_t)q[j * k + t] *
                            (int32_t)s_g[j * ng + t / group];
                double term = (double)a_scale[i * nb + b] * (double)part;
                sum += term;
                mag += fabs(term);
            }
            y[i * n + j] = sum * (double)s_ch[j];
            if (bound)
                bound[i * n + j] = mag * (double)s_ch[j];
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------- extension: W8A8 comparison path -- */

/* Reading R8: per-channel symmetric int8 weights, c = max |w|, s_ch = c/127. */
int oracle_quantize_w8_channel(const uint16_t *w, int64_t n, int64_t k, int8_t *q8,
                               float *s_ch)
{
    if (n < 0 || k < 0)
        return ORACLE_BAD_ARGS;
    if (n == 0)
        return ORACLE_OK;
    if (!w || !s_ch || (k > 0 && !q8))
        return ORACLE_BAD_ARGS;
    channel_int8(w, n, k, 127, q8, s_ch);
    return ORACLE_OK;
}

/* acc[m,n] = sum_k a_q[m,k] * q8[n,k] (int32), y = acc * s_a[m] * s_ch[n] (binary64). */
int oracle_w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *q8,
                     const float *s_ch, int64_t m, int64_t n, int64_t k, int32_t *acc,
                     double *y)
{
    if (m < 0 || n < 0 || k < 0 || k > ORACLE_K_MAX_127)
        return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int32_t total = 0;
            for (int64_t t = 0; t < k; ++t)
                total += (int32_t)a_q[i * k + t] * (int32_t)q8[j * k + t];
            if (acc)
                acc[i * n + j] = total;
            if (y)
                y[i * n + j] = (double)total * (double)a_scale[i] * (double)s_ch[j];
        }
    return ORACLE_OK;
}

/* ------------------------- extension: EQuARX local reduction step (R9) -- */

/*
 * One receive step of a block-quantized reduce-scatter ("EQuARX" verdict page,
 * pith_extraction.key_machinery: received blocks are dequantized to FP32 before
 * the partial-sum addition; the sum is block-quantized again for the next hop).
 *   d = fl(q_in * s_in);  v = fl(x + d)  with x binary32 (x_f32) or bf16 (x_bf16)
 *   (q_out, s_out) = block quantization of v (R1-R3 on binary32 input)
 * sum_out (may be NULL) receives v.  Exactly one of x_f32 / x_bf16 is given.
 */
int oracle_dequant_add_requant(const int8_t *q_in, const float *s_in, const float *x_f32,
                               const uint16_t *x_bf16, int64_t rows, int64_t cols,
                               int32_t block, float *sum_out, int8_t *q_out, float *s_out)
{
    if (rows < 0 || cols < 0 || block <= 0 || (cols % block) != 0 ||
        (x_f32 == NULL) == (x_bf16 == NULL))
        return ORACLE_BAD_ARGS;
    if (rows == 0 || cols == 0)
        return ORACLE_OK;
    if (!q_in || !s_in || !q_out || !s_out)
        return ORACLE_BAD_ARGS;
    const int64_t nblk = cols / block;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float *v = (float *)malloc(sizeof(float) * (size_t)block);
        for (int64_t b = 0; b < nblk; ++b) {
            const int64_t base = r * cols + b * block;
            const float sb = s_in[r * nblk + b];
            float amax = 0.0f;
            for (int32_t i = 0; i < block; ++i) {
                float d = (float)q_in[base + i] * sb;
                float x = x_f32 ? x_f32[base + i] : bf16_bits_to_float(x_bf16[base + i]);
                v[i] = x + d;
                float a = fabsf(v[i]);
                if (a > amax)
                    amax = a;
            }
            float s = amax / 127.0f;
            float inv = (amax > 0.0f) ? (127.0f / amax) : 0.0f;
            s_out[r * nblk + b] = s;
            for (int32_t i = 0; i < block; ++i) {
                q_out[base + i] = (int8_t)saturating_round_half_even(v[i] * inv, 127);
                if (sum_out)
                    sum_out[base + i] = v[i];
            }
        }
        free(v);
    }
    return ORACLE_OK;
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
