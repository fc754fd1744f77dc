// gemm_w4.hip -- the W4A8 GEMM on symmetric two-level 4-bit weights (layout V1,
// uint8 group scales): instantiation of gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace w4a8 {

hipError_t launch_w4a8_gemm(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                            const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                            int64_t n, int64_t k, void *out, int out_dtype,
                            hipStream_t stream, int32_t *partials) {
    return launch_gemm_fmt<kW4Sym>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k, out,
                                   out_dtype, stream, partials);
}

hipError_t launch_w4a8_gemm_bf16act(const uint16_t *a, const uint8_t *w_packed,
                                    const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                                    int64_t n, int64_t k, void *out, int out_dtype,
                                    int8_t *ws_q, float *ws_s, hipStream_t stream,
                                    int32_t *partials) {
    return launch_gemm_bf16act_fmt<kW4Sym>(a, w_packed, grp_scale, ch_scale, m, n, k, out,
                                           out_dtype, ws_q, ws_s, stream, partials);
}

size_t splitk_partial_bytes(int64_t m, int64_t n, int64_t k) {
    return splitk_workspace_bytes(m, n, k);
}

}  // namespace w4a8
