// abi.hip -- the extern "C" entry points of libw4a8.so (declared in w4a8.h):
// argument validation, variant choice and launch on the caller's stream.
// Nothing here allocates device memory.  The only state kept between calls is
// a per-device cache of the compute-unit count.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <vector>

#include "w4a8.h"
#include "launch.hpp"

namespace w4a8 {

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = -1;
    if (dev >= 0 && dev < kMaxDevices) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int ncu = 0;
    if (dev < 0 ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu <= 0)
        return 256;
    if (dev < kMaxDevices) cache[dev].store(ncu, std::memory_order_relaxed);
    return ncu;
}

}  // namespace w4a8

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool debug_sync_enabled() {
    const char *v = getenv("W4A8_DEBUG");
    return v && v[0] == '1';
}

// A floating point input of a call: device pointer, element count, bf16 or binary32.
struct FpInput {
    const void *p;
    size_t count;
    bool bf16;
};

// Debug mode only: wait for the stream (the inputs may still be being
// written), copy each floating point input to host memory in slices and look
// for NaN or Inf (all exponent bits set).  W4A8_OK outside debug mode.
w4a8_status debug_check_inputs(hipStream_t stream, std::initializer_list<FpInput> inputs) {
    if (!debug_sync_enabled()) return W4A8_OK;
    if (hipStreamSynchronize(stream) != hipSuccess) return W4A8_ERR_HIP;
    constexpr size_t kSlice = size_t(1) << 22;   // elements per host copy
    std::vector<uint32_t> host;
    for (const FpInput &in : inputs) {
        if (!in.p || in.count == 0) continue;
        const size_t esize = in.bf16 ? 2 : 4;
        for (size_t off = 0; off < in.count; off += kSlice) {
            const size_t cnt = in.count - off < kSlice ? in.count - off : kSlice;
            host.resize((cnt * esize + 3) / 4);
            if (hipMemcpy(host.data(), (const uint8_t *)in.p + off * esize, cnt * esize,
                          hipMemcpyDeviceToHost) != hipSuccess)
                return W4A8_ERR_HIP;
            if (in.bf16) {
                const uint16_t *h = (const uint16_t *)host.data();
                for (size_t i = 0; i < cnt; ++i)
                    if ((h[i] & 0x7f80u) == 0x7f80u) return W4A8_ERR_NONFINITE;
            } else {
                for (size_t i = 0; i < cnt; ++i)
                    if ((host[i] & 0x7f800000u) == 0x7f800000u) return W4A8_ERR_NONFINITE;
            }
        }
    }
    return W4A8_OK;
}

// Map a launch result to a status; with W4A8_DEBUG=1 also wait for the stream.
w4a8_status finish(hipError_t launched, hipStream_t stream) {
    if (launched != hipSuccess) return W4A8_ERR_HIP;
    if (debug_sync_enabled()) {
        if (hipStreamSynchronize(stream) != hipSuccess) return W4A8_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return W4A8_ERR_HIP;
    }
    return W4A8_OK;
}

w4a8_status check_act_shape(int64_t rows, int64_t cols, int32_t block) {
    if (rows < 0 || cols < 0 || block <= 0 || (block % 8) != 0 || (cols % block) != 0)
        return W4A8_ERR_SHAPE;
    return W4A8_OK;
}

w4a8_status check_weight_shape(int64_t n, int64_t k, int32_t group) {
    if (n < 0 || k < 0) return W4A8_ERR_SHAPE;
    if (group != W4A8_GROUP) return W4A8_ERR_UNSUPPORTED;
    if ((n % W4A8_N_TILE) != 0 || (k % W4A8_GROUP) != 0) return W4A8_ERR_SHAPE;
    return W4A8_OK;
}

// Shared checks of the GEMM entry points.  `a` is the activation pointer (int8
// codes or bf16); `a_scale` is only required when need_a_scale is set.
// grp_scale is the group parameter array of the 4-bit formats; formats without
// one (int8 weights) pass need_grp = false.  k_max is the format's int32 bound.
w4a8_status check_gemm_args(const void *a, const float *a_scale, bool need_a_scale,
                            const void *w_packed, const void *grp_scale,
                            const float *ch_scale, int64_t m, int64_t n, int64_t k,
                            int32_t group, const void *out, w4a8_dtype out_dtype,
                            int64_t k_max = W4A8_K_MAX, bool need_grp = true) {
    if (m < 0) return W4A8_ERR_SHAPE;
    w4a8_status st = check_weight_shape(n, k, group);
    if (st != W4A8_OK) return st;
    if (k > k_max) return W4A8_ERR_UNSUPPORTED;
    if (out_dtype != W4A8_F32 && out_dtype != W4A8_BF16 && out_dtype != W4A8_I32)
        return W4A8_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return W4A8_OK;
    const bool has_k = k > 0;
    if ((has_k && (!a || !w_packed || (need_grp && !grp_scale))) || !ch_scale || !out ||
        (need_a_scale && !a_scale))
        return W4A8_ERR_NULL;
    if ((has_k && (!aligned16(a) || !aligned16(w_packed) ||
                   (need_grp && !aligned16(grp_scale)))) ||
        !aligned16(ch_scale) || !aligned16(out) || (need_a_scale && !aligned16(a_scale)))
        return W4A8_ERR_MISALIGNED;
    return W4A8_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace checks of the fused entry points; on success sets the code and
// scale pointers inside it, and the split-K partials when the workspace also
// has w4a8_gemm_workspace_bytes(m, n, k) > 0 bytes after them (else null).
w4a8_status split_workspace(void *workspace, size_t ws_bytes, int64_t m, int64_t n, int64_t k,
                            int8_t **a_q, float **a_s, int32_t **partials) {
    if (!workspace) return W4A8_ERR_NULL;
    if (!aligned16(workspace)) return W4A8_ERR_MISALIGNED;
    const size_t base = w4a8_gemm_bf16act_workspace_bytes(m, k);
    if (ws_bytes < base) return W4A8_ERR_SHAPE;
    *a_q = (int8_t *)workspace;
    *a_s = (float *)((uint8_t *)workspace + round_up((size_t)m * (size_t)k, 256));
    const size_t extra = w4a8::splitk_partial_bytes(m, n, k);
    *partials = (extra > 0 && ws_bytes - base >= extra)
                    ? (int32_t *)((uint8_t *)workspace + base) : nullptr;
    return W4A8_OK;
}

}  // namespace

extern "C" {

int32_t w4a8_abi_version(void) { return W4A8_ABI_VERSION; }

int32_t w4a8_pack_layout_version(void) { return W4A8_PACK_LAYOUT_V1; }

const char *w4a8_status_string(w4a8_status status) {
    switch (status) {
        case W4A8_OK: return "ok";
        case W4A8_ERR_NULL: return "null pointer";
        case W4A8_ERR_SHAPE: return "invalid shape";
        case W4A8_ERR_UNSUPPORTED: return "unsupported argument";
        case W4A8_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case W4A8_ERR_HIP: return "HIP runtime error";
        case W4A8_ERR_NONFINITE: return "non-finite input (debug check)";
    }
    return "unknown status";
}

w4a8_status quantize_act_blockwise(const uint16_t *x, int64_t rows, int64_t cols, int32_t block,
                                   int8_t *q, float *scales, hipStream_t stream) {
    w4a8_status st = check_act_shape(rows, cols, block);
    if (st != W4A8_OK) return st;
    if (rows == 0 || cols == 0) return W4A8_OK;
    if (!x || !q || !scales) return W4A8_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(scales)) return W4A8_ERR_MISALIGNED;
    st = debug_check_inputs(stream, {{x, (size_t)(rows * cols), true}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_quantize_act(x, rows, cols, block, q, scales, stream), stream);
}

w4a8_status dequantize_act_blockwise(const int8_t *q, const float *scales, int64_t rows,
                                     int64_t cols, int32_t block, void *out,
                                     w4a8_dtype out_dtype, hipStream_t stream) {
    w4a8_status st = check_act_shape(rows, cols, block);
    if (st != W4A8_OK) return st;
    if (out_dtype != W4A8_F32 && out_dtype != W4A8_BF16) return W4A8_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return W4A8_OK;
    if (!q || !scales || !out) return W4A8_ERR_NULL;
    if (!aligned16(q) || !aligned16(scales) || !aligned16(out)) return W4A8_ERR_MISALIGNED;
    st = debug_check_inputs(stream, {{scales, (size_t)(rows * (cols / block)), false}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_dequantize_act(q, scales, rows, cols, block, out,
                                              out_dtype == W4A8_BF16, stream),
                  stream);
}

w4a8_status pack_w4_grouped(const uint16_t *w, int64_t n, int64_t k, int32_t group,
                            uint8_t *w_packed, uint8_t *grp_scale, float *ch_scale,
                            hipStream_t stream) {
    w4a8_status st = check_weight_shape(n, k, group);
    if (st != W4A8_OK) return st;
    if (n == 0) return W4A8_OK;
    if (!ch_scale || (k > 0 && (!w || !w_packed || !grp_scale))) return W4A8_ERR_NULL;
    if (!aligned16(ch_scale) ||
        (k > 0 && (!aligned16(w) || !aligned16(w_packed) || !aligned16(grp_scale))))
        return W4A8_ERR_MISALIGNED;
    st = debug_check_inputs(stream, {{w, (size_t)(n * k), true}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_pack_w4(w, n, k, w_packed, grp_scale, ch_scale, stream), stream);
}

w4a8_status unpack_w4_grouped(const uint8_t *w_packed, const uint8_t *grp_scale, int64_t n,
                              int64_t k, int32_t group, int8_t *q, uint8_t *s_g,
                              hipStream_t stream) {
    w4a8_status st = check_weight_shape(n, k, group);
    if (st != W4A8_OK) return st;
    if (n == 0 || k == 0) return W4A8_OK;
    if (!w_packed || !grp_scale || !q || !s_g) return W4A8_ERR_NULL;
    if (!aligned16(w_packed) || !aligned16(grp_scale) || !aligned16(q) || !aligned16(s_g))
        return W4A8_ERR_MISALIGNED;
    return finish(w4a8::launch_unpack_w4(w_packed, grp_scale, n, k, q, s_g, stream), stream);
}

w4a8_status w4a8_gemm(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                      const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                      int64_t k, int32_t group, void *out, w4a8_dtype out_dtype,
                      hipStream_t stream) {
    w4a8_status st = check_gemm_args(a_q, a_scale, true, w_packed, grp_scale, ch_scale, m, n,
                                     k, group, out, out_dtype);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a_scale, (size_t)m, false}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w4a8_gemm(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k,
                                         out, (int)out_dtype, stream),
                  stream);
}

size_t w4a8_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m <= 0 || n <= 0 || k <= 0) return 0;
    return w4a8::splitk_partial_bytes(m, n, k);
}

w4a8_status w4a8_gemm_ws(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                         const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                         int64_t k, int32_t group, void *out, w4a8_dtype out_dtype,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    w4a8_status st = check_gemm_args(a_q, a_scale, true, w_packed, grp_scale, ch_scale, m, n,
                                     k, group, out, out_dtype);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a_scale, (size_t)m, false}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    const size_t need = w4a8_gemm_workspace_bytes(m, n, k);
    int32_t *partials = nullptr;
    if (need > 0) {
        if (!workspace) return W4A8_ERR_NULL;
        if (!aligned16(workspace)) return W4A8_ERR_MISALIGNED;
        if (ws_bytes < need) return W4A8_ERR_SHAPE;
        partials = (int32_t *)workspace;
    }
    return finish(w4a8::launch_w4a8_gemm(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k,
                                         out, (int)out_dtype, stream, partials),
                  stream);
}

size_t w4a8_gemm_bf16act_workspace_bytes(int64_t m, int64_t k) {
    if (m <= 0 || k <= 0) return 0;
    return round_up((size_t)m * (size_t)k, 256) + round_up((size_t)m * sizeof(float), 256);
}

w4a8_status w4a8_gemm_bf16act(const uint16_t *a, const uint8_t *w_packed,
                              const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                              int64_t n, int64_t k, int32_t group, void *out,
                              w4a8_dtype out_dtype, void *workspace, size_t ws_bytes,
                              hipStream_t stream) {
    if (k <= 0 || m < 0) return W4A8_ERR_SHAPE;
    w4a8_status st = check_gemm_args(a, nullptr, false, w_packed, grp_scale, ch_scale, m, n,
                                     k, group, out, out_dtype);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a, (size_t)(m * k), true}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    int8_t *a_q;
    float *a_s;
    int32_t *partials;
    st = split_workspace(workspace, ws_bytes, m, n, k, &a_q, &a_s, &partials);
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w4a8_gemm_bf16act(a, w_packed, grp_scale, ch_scale, m, n, k, out,
                                                 (int)out_dtype, a_q, a_s, stream, partials),
                  stream);
}

/* ------------------------------------------------ LQQ (asymmetric) weights */

w4a8_status pack_w4_lqq(const uint16_t *w, int64_t n, int64_t k, int32_t group,
                        uint8_t *w_packed, uint16_t *grp_param, float *ch_scale,
                        hipStream_t stream) {
    w4a8_status st = check_weight_shape(n, k, group);
    if (st != W4A8_OK) return st;
    if (n == 0) return W4A8_OK;
    if (!ch_scale || (k > 0 && (!w || !w_packed || !grp_param))) return W4A8_ERR_NULL;
    if (!aligned16(ch_scale) ||
        (k > 0 && (!aligned16(w) || !aligned16(w_packed) || !aligned16(grp_param))))
        return W4A8_ERR_MISALIGNED;
    st = debug_check_inputs(stream, {{w, (size_t)(n * k), true}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_pack_w4_lqq(w, n, k, w_packed, grp_param, ch_scale, stream),
                  stream);
}

w4a8_status unpack_w4_lqq(const uint8_t *w_packed, const uint16_t *grp_param, int64_t n,
                          int64_t k, int32_t group, uint8_t *q_u4, uint8_t *s_u8,
                          int8_t *w_min, hipStream_t stream) {
    w4a8_status st = check_weight_shape(n, k, group);
    if (st != W4A8_OK) return st;
    if (n == 0 || k == 0) return W4A8_OK;
    if (!w_packed || !grp_param || !q_u4 || !s_u8 || !w_min) return W4A8_ERR_NULL;
    if (!aligned16(w_packed) || !aligned16(grp_param) || !aligned16(q_u4) || !aligned16(s_u8) ||
        !aligned16(w_min))
        return W4A8_ERR_MISALIGNED;
    return finish(w4a8::launch_unpack_w4_lqq(w_packed, grp_param, n, k, q_u4, s_u8, w_min,
                                             stream),
                  stream);
}

w4a8_status w4a8_gemm_lqq(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                          const uint16_t *grp_param, const float *ch_scale, int64_t m,
                          int64_t n, int64_t k, int32_t group, void *out, w4a8_dtype out_dtype,
                          hipStream_t stream) {
    w4a8_status st = check_gemm_args(a_q, a_scale, true, w_packed, grp_param, ch_scale, m, n,
                                     k, group, out, out_dtype, W4A8_LQQ_K_MAX);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a_scale, (size_t)m, false}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w4a8_gemm_lqq(a_q, a_scale, w_packed, grp_param, ch_scale, m, n,
                                             k, out, (int)out_dtype, stream),
                  stream);
}

w4a8_status w4a8_gemm_lqq_bf16act(const uint16_t *a, const uint8_t *w_packed,
                                  const uint16_t *grp_param, const float *ch_scale, int64_t m,
                                  int64_t n, int64_t k, int32_t group, void *out,
                                  w4a8_dtype out_dtype, void *workspace, size_t ws_bytes,
                                  hipStream_t stream) {
    if (k <= 0 || m < 0) return W4A8_ERR_SHAPE;
    w4a8_status st = check_gemm_args(a, nullptr, false, w_packed, grp_param, ch_scale, m, n, k,
                                     group, out, out_dtype, W4A8_LQQ_K_MAX);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a, (size_t)(m * k), true}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    int8_t *a_q;
    float *a_s;
    int32_t *partials;
    st = split_workspace(workspace, ws_bytes, m, n, k, &a_q, &a_s, &partials);
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w4a8_gemm_lqq_bf16act(a, w_packed, grp_param, ch_scale, m, n, k,
                                                     out, (int)out_dtype, a_q, a_s, stream, partials),
                  stream);
}

/* ---------------------------------------------------- W8A8 comparison path */

w4a8_status pack_w8_channel(const uint16_t *w, int64_t n, int64_t k, int8_t *w_packed,
                            float *ch_scale, hipStream_t stream) {
    w4a8_status st = check_weight_shape(n, k, W4A8_GROUP);
    if (st != W4A8_OK) return st;
    if (n == 0) return W4A8_OK;
    if (!ch_scale || (k > 0 && (!w || !w_packed))) return W4A8_ERR_NULL;
    if (!aligned16(ch_scale) || (k > 0 && (!aligned16(w) || !aligned16(w_packed))))
        return W4A8_ERR_MISALIGNED;
    st = debug_check_inputs(stream, {{w, (size_t)(n * k), true}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_pack_w8(w, n, k, w_packed, ch_scale, stream), stream);
}

w4a8_status unpack_w8_channel(const int8_t *w_packed, int64_t n, int64_t k, int8_t *q8,
                              hipStream_t stream) {
    w4a8_status st = check_weight_shape(n, k, W4A8_GROUP);
    if (st != W4A8_OK) return st;
    if (n == 0 || k == 0) return W4A8_OK;
    if (!w_packed || !q8) return W4A8_ERR_NULL;
    if (!aligned16(w_packed) || !aligned16(q8)) return W4A8_ERR_MISALIGNED;
    return finish(w4a8::launch_unpack_w8(w_packed, n, k, q8, stream), stream);
}

w4a8_status w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_packed,
                      const float *ch_scale, int64_t m, int64_t n, int64_t k, void *out,
                      w4a8_dtype out_dtype, hipStream_t stream) {
    w4a8_status st = check_gemm_args(a_q, a_scale, true, w_packed, nullptr, ch_scale, m, n, k,
                                     W4A8_GROUP, out, out_dtype, W4A8_LQQ_K_MAX, false);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a_scale, (size_t)m, false}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w8a8_gemm(a_q, a_scale, w_packed, ch_scale, m, n, k, out,
                                         (int)out_dtype, stream),
                  stream);
}

w4a8_status w8a8_gemm_bf16act(const uint16_t *a, const int8_t *w_packed, const float *ch_scale,
                              int64_t m, int64_t n, int64_t k, void *out, w4a8_dtype out_dtype,
                              void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (k <= 0 || m < 0) return W4A8_ERR_SHAPE;
    w4a8_status st = check_gemm_args(a, nullptr, false, w_packed, nullptr, ch_scale, m, n, k,
                                     W4A8_GROUP, out, out_dtype, W4A8_LQQ_K_MAX, false);
    if (st != W4A8_OK) return st;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream, {{a, (size_t)(m * k), true}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    int8_t *a_q;
    float *a_s;
    int32_t *partials;
    st = split_workspace(workspace, ws_bytes, m, n, k, &a_q, &a_s, &partials);
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w8a8_gemm_bf16act(a, w_packed, ch_scale, m, n, k, out,
                                                 (int)out_dtype, a_q, a_s, stream, partials),
                  stream);
}

/* -------------------------------------- per-block activation scales (GEMM) */

w4a8_status w4a8_gemm_blockact(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                               const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                               int64_t n, int64_t k, int32_t group, int32_t block, void *out,
                               w4a8_dtype out_dtype, hipStream_t stream) {
    if (block != 32 && block != 64 && block != 128) return W4A8_ERR_UNSUPPORTED;
    if (out_dtype == W4A8_I32) return W4A8_ERR_UNSUPPORTED;
    w4a8_status st = check_gemm_args(a_q, a_scale, true, w_packed, grp_scale, ch_scale, m, n,
                                     k, group, out, out_dtype);
    if (st != W4A8_OK) return st;
    if ((k % block) != 0) return W4A8_ERR_SHAPE;
    if (m == 0 || n == 0) return W4A8_OK;
    st = debug_check_inputs(stream,
                            {{a_scale, (size_t)(m * (k / block)), false}, {ch_scale, (size_t)n, false}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_w4a8_gemm_blockact(a_q, a_scale, w_packed, grp_scale, ch_scale, m,
                                                  n, k, block, out, (int)out_dtype, stream),
                  stream);
}

/* ------------------------------------------------- EQuARX receive step */

w4a8_status dequant_add_requant(const int8_t *q_in, const float *s_in, const void *x,
                                w4a8_dtype x_dtype, int64_t rows, int64_t cols, int32_t block,
                                float *sum_out, int8_t *q_out, float *s_out,
                                hipStream_t stream) {
    w4a8_status st = check_act_shape(rows, cols, block);
    if (st != W4A8_OK) return st;
    if (x_dtype != W4A8_F32 && x_dtype != W4A8_BF16) return W4A8_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return W4A8_OK;
    if (!q_in || !s_in || !x || !q_out || !s_out) return W4A8_ERR_NULL;
    if (!aligned16(q_in) || !aligned16(s_in) || !aligned16(x) || !aligned16(q_out) ||
        !aligned16(s_out) || (sum_out && !aligned16(sum_out)))
        return W4A8_ERR_MISALIGNED;
    st = debug_check_inputs(stream, {{s_in, (size_t)(rows * (cols / block)), false},
                                     {x, (size_t)(rows * cols), x_dtype == W4A8_BF16}});
    if (st != W4A8_OK) return st;
    return finish(w4a8::launch_dequant_add_requant(q_in, s_in, x, x_dtype == W4A8_BF16, rows,
                                                   cols, block, sum_out, q_out, s_out, stream),
                  stream);
}

/* ------------------------------------------------------ measurement aid */

w4a8_status w4a8_probe_mfma_i8(int64_t workgroups, int32_t iters, int32_t *sink,
                               uint64_t *clocks, hipStream_t stream) {
    if (workgroups < 1 || workgroups > 65535 || iters < 1) return W4A8_ERR_SHAPE;
    if (!sink || !clocks) return W4A8_ERR_NULL;
    if (!aligned16(sink) || !aligned16(clocks)) return W4A8_ERR_MISALIGNED;
    return finish(w4a8::launch_mfma_probe(workgroups, iters, sink, clocks, stream), stream);
}

}  // extern "C"
