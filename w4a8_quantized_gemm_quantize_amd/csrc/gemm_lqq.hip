// gemm_lqq.hip -- the W4A8 GEMM on LiquidGEMM's asymmetric LQQ weights (layout
// V1 nibbles, uint16 group parameters s | (128 + min) << 8): instantiation of
// gemm_kernels.hpp.  The rebuilt operand u s + min is still int8, so the MFMA
// core and the exact int32 accumulation are unchanged.
#include "gemm_kernels.hpp"

namespace w4a8 {

hipError_t launch_w4a8_gemm_lqq(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                                const uint16_t *grp_param, const float *ch_scale, int64_t m,
                                int64_t n, int64_t k, void *out, int out_dtype,
                                hipStream_t stream, int32_t *partials) {
    return launch_gemm_fmt<kW4Lqq>(a_q, a_scale, w_packed, (const uint8_t *)grp_param,
                                   ch_scale, m, n, k, out, out_dtype, stream, partials);
}

hipError_t launch_w4a8_gemm_lqq_bf16act(const uint16_t *a, const uint8_t *w_packed,
                                        const uint16_t *grp_param, const float *ch_scale,
                                        int64_t m, int64_t n, int64_t k, void *out,
                                        int out_dtype, int8_t *ws_q, float *ws_s,
                                        hipStream_t stream, int32_t *partials) {
    return launch_gemm_bf16act_fmt<kW4Lqq>(a, w_packed, (const uint8_t *)grp_param, ch_scale, m,
                                           n, k, out, out_dtype, ws_q, ws_s, stream, partials);
}

}  // namespace w4a8
