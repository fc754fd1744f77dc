// gemm_w8.hip -- the W8A8 comparison GEMM: per-channel int8 weights (kW8 layout)
// on the same MFMA core, staging and epilogue as the W4A8 kernels, with the
// 4-bit rebuild replaced by the stored int8 operand: instantiation of
// gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace w4a8 {

hipError_t launch_w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_packed,
                            const float *ch_scale, int64_t m, int64_t n, int64_t k, void *out,
                            int out_dtype, hipStream_t stream, int32_t *partials) {
    return launch_gemm_fmt<kW8>(a_q, a_scale, (const uint8_t *)w_packed, nullptr, ch_scale, m,
                                n, k, out, out_dtype, stream, partials);
}

hipError_t launch_w8a8_gemm_bf16act(const uint16_t *a, const int8_t *w_packed,
                                    const float *ch_scale, int64_t m, int64_t n, int64_t k,
                                    void *out, int out_dtype, int8_t *ws_q, float *ws_s,
                                    hipStream_t stream, int32_t *partials) {
    return launch_gemm_bf16act_fmt<kW8>(a, (const uint8_t *)w_packed, nullptr, ch_scale, m, n, k,
                                        out, out_dtype, ws_q, ws_s, stream, partials);
}

}  // namespace w4a8
