// gemm_blockact.hip -- the W4A8 GEMM with per-block activation scales (blocks
// of 32, 64 or 128 along K, as written by quantize_act_blockwise): the int32
// partial of each activation block comes out of the MFMA exactly and is folded
// into a binary32 accumulator with that block's scale, block after block in K
// order; the channel scale is applied at the end.  Symmetric 4-bit weights
// (layout V1); instantiation of gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace w4a8 {

hipError_t launch_w4a8_gemm_blockact(const int8_t *a_q, const float *a_scale,
                                     const uint8_t *w_packed, const uint8_t *grp_scale,
                                     const float *ch_scale, int64_t m, int64_t n, int64_t k,
                                     int32_t block, void *out, int out_dtype,
                                     hipStream_t stream) {
    switch (block) {
        case 32:
            return launch_gemm_blockact_fmt<kW4Sym, 32>(a_q, a_scale, w_packed, grp_scale,
                                                        ch_scale, m, n, k, out, out_dtype, stream);
        case 64:
            return launch_gemm_blockact_fmt<kW4Sym, 64>(a_q, a_scale, w_packed, grp_scale,
                                                        ch_scale, m, n, k, out, out_dtype, stream);
        case 128:
            return launch_gemm_blockact_fmt<kW4Sym, 128>(a_q, a_scale, w_packed, grp_scale,
                                                         ch_scale, m, n, k, out, out_dtype,
                                                         stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace w4a8
