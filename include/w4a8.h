/*
 * w4a8.h -- C ABI of libw4a8.so: block-scaled int8 activation quantization
 * and a W4A8 grouped GEMM for AMD Instinct MI355X (gfx950).
 *
 * Method (pages cited by title and section):
 *   - Activations: block-wise symmetric int8 with one binary32 scale per block
 *     taken from the block's absolute maximum, computed in two phases (scales,
 *     then scaled data), dequantized back to binary32.
 *     ["EQuARX" verdict page, pith.science arXiv 2506.17615,
 *      pith_extraction.key_machinery]
 *   - Weights: two levels -- an INT8 first level per output channel with a
 *     protective range, then 4-bit codes with a small integer scale per group
 *     of 64 along K, so that rebuilding the int8 operand is one multiply-add
 *     and one XOR per four weights.
 *     ["LiquidGEMM" verdict page, pith.science arXiv 2509.01229,
 *      referee_report.summary, pith_extraction.key_machinery,
 *      referee_report.major_comments[2] (paper section 4, Eq. 7),
 *      skeptic_critique.concrete_test (group size 64)]
 *   - GEMM: int8 x int8 products accumulated exactly in int32, the integer
 *     group scale applied per K-group (folded into the int8 weight operand),
 *     then out = acc * a_scale[m] * ch_scale[n] in binary32.
 *     ["LiquidGEMM" verdict page, referee_report.summary: INT8 MMA into
 *      INT32 after in-kernel dequantization]
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers into caller-owned memory.  The library
 *     never allocates or frees device memory and keeps no global state; it is
 *     safe to call from several host threads.
 *   - Tensors are row-major and contiguous; bf16 is passed as its 16-bit
 *     pattern (uint16_t).
 *   - Every pointer must be 16-byte aligned (W4A8_ERR_MISALIGNED otherwise).
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronizing.
 *   - Argument errors are detected before anything is launched; then nothing
 *     is written and a non-zero status is returned.  A failed launch returns
 *     W4A8_ERR_HIP.  Faults during execution surface at the caller's next
 *     synchronization.
 *   - Empty inputs (rows == 0, m == 0, n == 0) are valid and do nothing.
 *   - NaN or infinite inputs are outside the contract (results unspecified).
 *   - Debug mode (environment variable W4A8_DEBUG=1, read on every call):
 *     before launching, a call synchronizes its stream, copies its floating
 *     point inputs (bf16 activations or weights, binary32 scales or partial
 *     sums) to host memory and returns W4A8_ERR_NONFINITE, writing nothing, if
 *     any element is NaN or infinite; after launching it synchronizes again and
 *     reports execution errors as W4A8_ERR_HIP.  Debug mode is slow (host
 *     scans) and meant for development only.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A8_ABI_VERSION 1
#define W4A8_PACK_LAYOUT_V1 1
/* Weight group size along K (the only supported value). */
#define W4A8_GROUP 64
/* Output channels are packed in tiles of 16; n must be a multiple of it. */
#define W4A8_N_TILE 16
/* Largest K for which |acc| <= K * 127 * 112 fits in int32. */
#define W4A8_K_MAX 150976
/* Weight codes: level-1 protective range and level-2 code range. */
#define W4A8_W8_RANGE 112
#define W4A8_W4_RANGE 7

typedef enum {
    W4A8_OK = 0,
    W4A8_ERR_NULL = 1,        /* a required pointer is NULL */
    W4A8_ERR_SHAPE = 2,       /* negative size or a divisibility rule is broken */
    W4A8_ERR_UNSUPPORTED = 3, /* valid request this build does not implement */
    W4A8_ERR_MISALIGNED = 4,  /* a pointer is not 16-byte aligned */
    W4A8_ERR_HIP = 5,         /* the HIP runtime reported an error */
    W4A8_ERR_NONFINITE = 6    /* debug mode only: a floating point input holds NaN or Inf */
} w4a8_status;

typedef enum {
    W4A8_F32 = 0,  /* binary32 output */
    W4A8_BF16 = 1, /* bf16 output: round-to-nearest-even of the binary32 value */
    W4A8_I32 = 2   /* raw int32 accumulator acc[m,n] (GEMM only; exact) */
} w4a8_dtype;

/* W4A8_ABI_VERSION of the loaded library. */
int32_t w4a8_abi_version(void);

/* W4A8_PACK_LAYOUT_V1: version of the packed weight layout this library writes and reads. */
int32_t w4a8_pack_layout_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *w4a8_status_string(w4a8_status status);

/*
 * Block-wise int8 quantization of activations ("EQuARX" verdict page,
 * pith_extraction.key_machinery: absmax per block, one binary32 scale per
 * block, scale then round).
 *   x      [rows, cols] bf16 (input)
 *   q      [rows, cols] int8 (output), codes in [-127, 127]
 *   scales [rows, cols/block] binary32 (output)
 * Per block of `block` contiguous elements of a row:
 *   amax = max |x|,  s = amax / 127,  inv = (amax > 0) ? 127 / amax : 0,
 *   q = clamp(round_half_even(x * inv), -127, 127) with x * inv one binary32
 *   multiply; a NaN product (0 * inf when 127/amax overflows) gives 0.
 * Requires block > 0, block % 8 == 0 and cols % block == 0 (W4A8_ERR_SHAPE).
 * block == cols gives one scale per row (per token).
 */
w4a8_status quantize_act_blockwise(const uint16_t *x, int64_t rows, int64_t cols, int32_t block,
                                   int8_t *q, float *scales, hipStream_t stream);

/*
 * Dequantization back to binary32 ("EQuARX" verdict page,
 * pith_extraction.key_machinery: dequantize to FP32).
 *   out[r, c] = q[r, c] * scales[r, c / block]   (one binary32 multiply)
 * out_dtype W4A8_F32 writes float [rows, cols]; W4A8_BF16 writes the bf16
 * rounding (nearest-even) of that value as uint16_t [rows, cols].
 * W4A8_I32 is W4A8_ERR_UNSUPPORTED.  Shape rules as for quantize_act_blockwise.
 */
w4a8_status dequantize_act_blockwise(const int8_t *q, const float *scales, int64_t rows,
                                     int64_t cols, int32_t block, void *out,
                                     w4a8_dtype out_dtype, hipStream_t stream);

/*
 * Two-level 4-bit weight quantization and packing ("LiquidGEMM" verdict
 * page, referee_report.summary: INT8 first level, then 4-bit with an integer
 * group scale; referee_report.major_comments[2]: the group scale is at most 16).
 *   w         [n, k] bf16, nn.Linear layout (output channel major) (input)
 *   w_packed  n * k / 2 bytes, packed layout V1 (output, opaque)
 *   grp_scale n * k / 64 bytes, uint8 group scales in kernel order (output)
 *   ch_scale  [n] binary32 per-channel scales (output)
 * Per channel: c = max |w|, ch_scale = c / 112,
 *   W8 = clamp(round_half_even(w * (112 / c)), -112, 112)  (0 when c == 0).
 * Per group of 64 along k: m = max |W8|, s_g = max(1, ceil(m / 7)) in [1, 16],
 *   q = round_half_even(W8 / s_g) in [-7, 7] (exact rational rounding),
 *   stored as the nibble q + 8.
 * The effective weight is ch_scale[n] * s_g[n, g] * q[n, k].
 * Requires group == 64 (else W4A8_ERR_UNSUPPORTED), n % 16 == 0 and
 * k % 64 == 0 (else W4A8_ERR_SHAPE).  This step is run once per weight.
 */
w4a8_status pack_w4_grouped(const uint16_t *w, int64_t n, int64_t k, int32_t group,
                            uint8_t *w_packed, uint8_t *grp_scale, float *ch_scale,
                            hipStream_t stream);

/*
 * Inverse of the packing (test hook): decodes layout V1 back to canonical
 * codes q [n, k] int8 in [-7, 7] and group scales s_g [n, k / 64] uint8 in
 * plain row-major order.  Shape rules as for pack_w4_grouped.
 */
w4a8_status unpack_w4_grouped(const uint8_t *w_packed, const uint8_t *grp_scale, int64_t n,
                              int64_t k, int32_t group, int8_t *q, uint8_t *s_g,
                              hipStream_t stream);

/*
 * W4A8 GEMM with per-token activation scales.
 *   a_q       [m, k] int8 activation codes
 *   a_scale   [m] binary32 per-row activation scales
 *   w_packed, grp_scale, ch_scale: as written by pack_w4_grouped for [n, k]
 *   out       [m, n]: W4A8_F32 float, W4A8_BF16 uint16_t, W4A8_I32 int32_t
 * acc[m, n] = sum_g s_g[n, g] * sum_{k in g} a_q[m, k] * q[n, k]   (int32, exact)
 * out[m, n] = (float(acc) * a_scale[m]) * ch_scale[n]              (binary32),
 *             rounded to bf16 (nearest-even) for W4A8_BF16; W4A8_I32 stores acc.
 * Requires group == 64, n % 16 == 0, k % 64 == 0 and k <= W4A8_K_MAX
 * (larger k is W4A8_ERR_UNSUPPORTED).  k == 0 writes zeros.
 */
w4a8_status w4a8_gemm(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                      const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                      int64_t k, int32_t group, void *out, w4a8_dtype out_dtype,
                      hipStream_t stream);

/*
 * Bytes of optional scratch that lets w4a8_gemm_ws (and the fused entry points
 * below) split K over workgroups for an m x n x k product: int32 partial sums,
 * (S slices of m * n int32, S from 2 to 16).  Split shapes:
 *   - 5 <= m <= 64 (the one-pass kernel re-reads all of A in every
 *     workgroup): S = min(ceil(512 / ceil(n / 128)), 16), cut to keep the
 *     partials within half the weight bytes (32 * S * m <= k); for m > 16
 *     with no cut always split, otherwise where a model of the two paths'
 *     times, fitted to MI355X measurements, favours the split;
 *   - m > 64 with at most 128 output tiles of 128 x 256 (the one-pass kernels
 *     would leave CUs idle), S = min(256 / tiles, k / (8 m)), or up to
 *     64 MiB of partials when k >= 4096 (k >= 2048 with at most 32 tiles),
 *     with slices of at least four 128-wide chunks.
 * 0 when the shape is not split (also for fewer than two 128-wide chunks of
 * K).  Part of the GEMM design choices, not of the method: the
 * result is the same bit for bit.
 */
size_t w4a8_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/*
 * w4a8_gemm with an optional workspace (16-byte aligned device memory owned by
 * the caller, contents undefined on entry and after the call).  When
 * w4a8_gemm_workspace_bytes(m, n, k) > 0 the workspace is required
 * (W4A8_ERR_NULL / W4A8_ERR_MISALIGNED / W4A8_ERR_SHAPE if null, misaligned or
 * smaller) and the product splits K; otherwise it is ignored and may be null.
 * Same arguments, rules and result as w4a8_gemm.  Calls that share a workspace
 * must be ordered (one stream).
 */
w4a8_status w4a8_gemm_ws(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                         const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                         int64_t k, int32_t group, void *out, w4a8_dtype out_dtype,
                         void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of workspace w4a8_gemm_bf16act needs for m rows of k activations:
 * the int8 codes [m, k] at offset 0, then the binary32 per-row scales [m] at
 * offset round_up(m * k, 256).
 */
size_t w4a8_gemm_bf16act_workspace_bytes(int64_t m, int64_t k);

/*
 * Fused entry point from bf16 activations: per-token quantization
 * (quantize_act_blockwise with block == k) into `workspace`, then w4a8_gemm.
 * The result equals those two calls bit for bit; the workspace holds the
 * activation codes and scales afterwards (layout above).  ws_bytes must be
 * at least w4a8_gemm_bf16act_workspace_bytes(m, k) (W4A8_ERR_SHAPE).  When it
 * also has w4a8_gemm_workspace_bytes(m, n, k) > 0 bytes after that, they hold
 * the split-K partials (as for w4a8_gemm_ws).
 * Requires k > 0 and the w4a8_gemm shape rules.
 */
w4a8_status w4a8_gemm_bf16act(const uint16_t *a, const uint8_t *w_packed,
                              const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                              int64_t n, int64_t k, int32_t group, void *out,
                              w4a8_dtype out_dtype, void *workspace, size_t ws_bytes,
                              hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as w4a8_gemm_bf16act, same arguments, rules and result bit for bit,
 * with its workspace (activation codes and scales, and the split-K partials
 * when the shape splits) in a static device array of the library instead of
 * caller memory.  Nothing is allocated or freed by the call; the caller passes
 * the inputs and `out` as usual.
 *   - The array holds W4A8_NOALLOC_SCRATCH_BYTES (64 MiB) per device, placed
 *     when the library's code is loaded on that device and kept until the
 *     process ends.  A call whose activation codes and scales would exceed
 *     it, w4a8_gemm_bf16act_workspace_bytes(m, k) >
 *     W4A8_NOALLOC_SCRATCH_BYTES, returns W4A8_ERR_UNSUPPORTED before
 *     touching the device (the 70B FFN-down shapes up to m = 2048 fit).  When
 *     the codes fit but the split-K partials, w4a8_gemm_workspace_bytes(m, n,
 *     k) more, do not, K is not split (same result bit for bit).
 *   - Every call on a device shares that device's array and leaves its
 *     contents behind: calls that overlap on one device (two streams, two
 *     host threads) race and must be ordered by the caller.
 *   - The array's address is looked up once per device, on the first call
 *     with that device current (W4A8_ERR_HIP if that fails).
 */
#define W4A8_NOALLOC_SCRATCH_BYTES (64ll << 20)
w4a8_status w4a8_gemm_bf16act_noalloc(const uint16_t *a, const uint8_t *w_packed,
                                      const uint8_t *grp_scale, const float *ch_scale,
                                      int64_t m, int64_t n, int64_t k, int32_t group, void *out,
                                      w4a8_dtype out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * LQQ weights: LiquidGEMM's own asymmetric 4-bit format ("LiquidGEMM" verdict
 * page, pith_extraction.key_machinery: INT8 weights shifted by the group
 * minimum into the unsigned domain, 4-bit codes with an integer scale, and the
 * rebuild (q_u4 * s_u8 + a) XOR 0x80 with a = 128 + min;
 * referee_report.major_comments[2] (paper section 4, Eq. 7): protective range
 * 119 and s_u8 <= 16).
 * ------------------------------------------------------------------------ */

/* Largest K for which |acc| <= K * 127 * 127 fits in int32 (multiple of 64):
 * the bound when weight operands reach 127 (LQQ and int8 weights). */
#define W4A8_LQQ_K_MAX 133120

/*
 * LQQ quantization and packing.
 *   w         [n, k] bf16 (input)
 *   w_packed  n * k / 2 bytes, layout V1 (nibble = q_u4) (output)
 *   grp_param n * k / 64 uint16, kernel order like grp_scale:
 *             s_u8 | (128 + min) << 8 (output)
 *   ch_scale  [n] binary32 (output)
 * Per channel: c = max |w|, ch_scale = c / 119,
 *   Q = clamp(round_half_even(w * (119 / c)), -119, 119)  (0 when c == 0).
 * Per group of 64: min, max of Q; s_u8 = max(1, nearest integer to
 *   (max - min) / 15) in [1, 16]; q_u4 = min(15, round_half_even((Q - min) / s_u8)).
 * Effective weight: ch_scale[n] * (q_u4 * s_u8 + min); the int8 operand
 * q_u4 * s_u8 + min lies in [-119, 127].  Shape rules as for pack_w4_grouped.
 */
w4a8_status pack_w4_lqq(const uint16_t *w, int64_t n, int64_t k, int32_t group,
                        uint8_t *w_packed, uint16_t *grp_param, float *ch_scale,
                        hipStream_t stream);

/* Inverse (test hook): q_u4 [n, k] uint8 in [0, 15], s_u8 [n, k/64] uint8,
 * w_min [n, k/64] int8, all plain row-major. */
w4a8_status unpack_w4_lqq(const uint8_t *w_packed, const uint16_t *grp_param, int64_t n,
                          int64_t k, int32_t group, uint8_t *q_u4, uint8_t *s_u8,
                          int8_t *w_min, hipStream_t stream);

/*
 * W4A8 GEMM on LQQ weights, per-token activation scales:
 *   acc[m, n] = sum_k a_q[m, k] * (q_u4[n, k] * s_u8[n, g] + min[n, g])  (int32, exact)
 *   out as for w4a8_gemm.  Requires k <= W4A8_LQQ_K_MAX and the w4a8_gemm rules.
 */
w4a8_status w4a8_gemm_lqq(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                          const uint16_t *grp_param, const float *ch_scale, int64_t m,
                          int64_t n, int64_t k, int32_t group, void *out, w4a8_dtype out_dtype,
                          hipStream_t stream);

/* Fused per-token quantization + w4a8_gemm_lqq (workspace as for w4a8_gemm_bf16act). */
w4a8_status w4a8_gemm_lqq_bf16act(const uint16_t *a, const uint8_t *w_packed,
                                  const uint16_t *grp_param, const float *ch_scale, int64_t m,
                                  int64_t n, int64_t k, int32_t group, void *out,
                                  w4a8_dtype out_dtype, void *workspace, size_t ws_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * W8A8 comparison path: per-channel symmetric int8 weights on the same MFMA
 * core, to test the regime claim of the "LiquidGEMM" verdict page
 * (pith_extraction.forward_implications: W4A8 wins when memory-bound and
 * matches W8A8 when compute-bound).
 * ------------------------------------------------------------------------ */

/*
 * w [n, k] bf16 -> w_packed n * k bytes (int8, opaque tiled layout),
 * ch_scale [n] binary32.  Per channel: c = max |w|, ch_scale = c / 127,
 * q8 = clamp(round_half_even(w * (127 / c)), -127, 127).
 * Requires n % 16 == 0 and k % 64 == 0.
 */
w4a8_status pack_w8_channel(const uint16_t *w, int64_t n, int64_t k, int8_t *w_packed,
                            float *ch_scale, hipStream_t stream);

/* Inverse (test hook): q8 [n, k] int8, row-major. */
w4a8_status unpack_w8_channel(const int8_t *w_packed, int64_t n, int64_t k, int8_t *q8,
                              hipStream_t stream);

/*
 * acc[m, n] = sum_k a_q[m, k] * q8[n, k] (int32, exact);
 * out[m, n] = (float(acc) * a_scale[m]) * ch_scale[n], as for w4a8_gemm.
 * Requires n % 16 == 0, k % 64 == 0, k <= W4A8_LQQ_K_MAX.
 */
w4a8_status w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_packed,
                      const float *ch_scale, int64_t m, int64_t n, int64_t k, void *out,
                      w4a8_dtype out_dtype, hipStream_t stream);

/* Fused per-token quantization + w8a8_gemm (workspace as for w4a8_gemm_bf16act). */
w4a8_status w8a8_gemm_bf16act(const uint16_t *a, const int8_t *w_packed, const float *ch_scale,
                              int64_t m, int64_t n, int64_t k, void *out, w4a8_dtype out_dtype,
                              void *workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-block activation scales inside the GEMM: activations quantized by
 * quantize_act_blockwise with blocks of 32, 64 or 128 along K ("EQuARX"
 * verdict page, pith_extraction.key_machinery: one FP32 scale per block) feed
 * the W4A8 GEMM directly; the block scales are applied per K-group as the
 * int32 partials come out of the matrix cores.
 * ------------------------------------------------------------------------ */

/*
 *   a_q      [m, k] int8, a_scale [m, k / block] binary32 (quantize_act_blockwise
 *            output with the same block)
 *   w_packed, grp_scale, ch_scale: as written by pack_w4_grouped
 *   out      [m, n] binary32 (W4A8_F32) or bf16 (W4A8_BF16); W4A8_I32 is
 *            W4A8_ERR_UNSUPPORTED
 * For each activation block b (k in [b * block, (b + 1) * block)):
 *   P_b[m, n] = sum_{k in b} a_q[m, k] * q[n, k] * s_g[n, k / 64]   (int32, exact)
 * and, in binary32 with blocks in increasing order (the order within one
 * block's row of a wavefront's K range; ranges of different wavefronts may be
 * summed in another order), each block folded by one fused multiply-add (one
 * rounding):
 *   f = 0;  f = fma(P_b, a_scale[m, b], f)  for each b;   out = f * ch_scale[n].
 * The error against the exact value is at most about (k / block + 2) * 2^-24
 * times sum_b |a_scale[m, b] * P_b| * ch_scale[n].
 * block must be 32, 64 or 128 (else W4A8_ERR_UNSUPPORTED) and divide k
 * (W4A8_ERR_SHAPE); otherwise the w4a8_gemm rules apply.
 */
w4a8_status w4a8_gemm_blockact(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                               const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                               int64_t n, int64_t k, int32_t group, int32_t block, void *out,
                               w4a8_dtype out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * EQuARX receive step ("EQuARX" verdict page, pith_extraction.key_machinery:
 * a block-quantized int8 shard is dequantized to FP32 before it is added to
 * the local partial sum, and the sum is block-quantized again for the next
 * hop of the ring).  The single-GPU local step of that reduction.
 * ------------------------------------------------------------------------ */

/*
 *   q_in    [rows, cols] int8 and s_in [rows, cols/block] binary32: the
 *           received block-quantized shard
 *   x       [rows, cols] local partial sum: binary32 (x_dtype W4A8_F32) or
 *           bf16 bits (W4A8_BF16)
 *   sum_out [rows, cols] binary32, may be NULL: v = fl(x + fl(q_in * s_in))
 *   q_out, s_out: quantize_act_blockwise of v (same block, same rounding:
 *           s = amax / 127, q = rne(v * (127 / amax)) in [-127, 127])
 * Shape rules as for quantize_act_blockwise; x_dtype W4A8_I32 is
 * W4A8_ERR_UNSUPPORTED.  q_out may not alias q_in; sum_out may not alias x.
 */
w4a8_status dequant_add_requant(const int8_t *q_in, const float *s_in, const void *x,
                                w4a8_dtype x_dtype, int64_t rows, int64_t cols, int32_t block,
                                float *sum_out, int8_t *q_out, float *s_out,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not part of the method): the int8 matrix-core reference
 * that the GEMMs' utilisation is compared with, and the shader clock.
 * ------------------------------------------------------------------------ */

/*
 * Runs `workgroups` workgroups of 8 wavefronts (two per SIMD with one per
 * compute unit); each wavefront does `iters` rounds of 16 independent
 * v_mfma_i32_16x16x64_i8 products, i.e. workgroups * iters * 4,194,304 int8
 * operations (a multiply-add counts 2) and nothing else.
 *   sink    int32 [workgroups * 512] (output; the accumulators' sums, so the
 *           loop is not removed)
 *   clocks  uint64 [2] (output): shader clock counter ticks (s_memtime) and
 *           100 MHz real-time ticks (s_memrealtime) over one wavefront's loop;
 *           clock (Hz) = clocks[0] / clocks[1] * 1e8.
 * Requires workgroups in [1, 65535] and iters >= 1 (W4A8_ERR_SHAPE).
 */
w4a8_status w4a8_probe_mfma_i8(int64_t workgroups, int32_t iters, int32_t *sink,
                               uint64_t *clocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
