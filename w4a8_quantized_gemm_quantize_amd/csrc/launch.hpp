// launch.hpp -- internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

// Compute units of the current device, queried once per device and cached
// (the launchers size grids by it on every call).
int device_cu_count();

hipError_t launch_quantize_act(const uint16_t *x, int64_t rows, int64_t cols, int32_t block,
                               int8_t *q, float *scales, hipStream_t stream);
hipError_t launch_dequantize_act(const int8_t *q, const float *scales, int64_t rows,
                                 int64_t cols, int32_t block, void *out, bool bf16,
                                 hipStream_t stream);
hipError_t launch_pack_w4(const uint16_t *w, int64_t n, int64_t k, uint8_t *w_packed,
                          uint8_t *grp_scale, float *ch_scale, hipStream_t stream);
hipError_t launch_unpack_w4(const uint8_t *w_packed, const uint8_t *grp_scale, int64_t n,
                            int64_t k, int8_t *q, uint8_t *s_g, hipStream_t stream);
// out_dtype: 0 = binary32, 1 = bf16, 2 = int32 accumulator.
// partials (optional, splitk_partial_bytes(m, n, k) bytes, 16-byte aligned):
// int32 scratch that lets batches whose output tiles would not fill the GPU
// split K over workgroups (splitk_slices); without it those
// shapes run the one-pass kernels.  Same result bit for bit either way.
size_t splitk_partial_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_w4a8_gemm(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                            const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                            int64_t n, int64_t k, void *out, int out_dtype, hipStream_t stream,
                            int32_t *partials = nullptr);
// Per-token quantization of bf16 activations into (ws_q, ws_s) and the GEMM;
// small m runs both in one kernel.
hipError_t launch_w4a8_gemm_bf16act(const uint16_t *a, const uint8_t *w_packed,
                                    const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                                    int64_t n, int64_t k, void *out, int out_dtype,
                                    int8_t *ws_q, float *ws_s, hipStream_t stream,
                                    int32_t *partials = nullptr);


// LiquidGEMM's asymmetric LQQ weights (parameter s | (128 + min) << 8 per group).
hipError_t launch_pack_w4_lqq(const uint16_t *w, int64_t n, int64_t k, uint8_t *w_packed,
                              uint16_t *grp_param, float *ch_scale, hipStream_t stream);
hipError_t launch_unpack_w4_lqq(const uint8_t *w_packed, const uint16_t *grp_param, int64_t n,
                                int64_t k, uint8_t *q_u4, uint8_t *s_u8, int8_t *w_min,
                                hipStream_t stream);
hipError_t launch_w4a8_gemm_lqq(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                                const uint16_t *grp_param, const float *ch_scale, int64_t m,
                                int64_t n, int64_t k, void *out, int out_dtype,
                                hipStream_t stream, int32_t *partials = nullptr);
hipError_t launch_w4a8_gemm_lqq_bf16act(const uint16_t *a, const uint8_t *w_packed,
                                        const uint16_t *grp_param, const float *ch_scale,
                                        int64_t m, int64_t n, int64_t k, void *out,
                                        int out_dtype, int8_t *ws_q, float *ws_s,
                                        hipStream_t stream, int32_t *partials = nullptr);

// W8A8 comparison path: per-channel int8 weights in the kW8 layout.
hipError_t launch_pack_w8(const uint16_t *w, int64_t n, int64_t k, int8_t *w_packed,
                          float *ch_scale, hipStream_t stream);
hipError_t launch_unpack_w8(const int8_t *w_packed, int64_t n, int64_t k, int8_t *q8,
                            hipStream_t stream);
hipError_t launch_w8a8_gemm(const int8_t *a_q, const float *a_scale, const int8_t *w_packed,
                            const float *ch_scale, int64_t m, int64_t n, int64_t k, void *out,
                            int out_dtype, hipStream_t stream, int32_t *partials = nullptr);
hipError_t launch_w8a8_gemm_bf16act(const uint16_t *a, const int8_t *w_packed,
                                    const float *ch_scale, int64_t m, int64_t n, int64_t k,
                                    void *out, int out_dtype, int8_t *ws_q, float *ws_s,
                                    hipStream_t stream, int32_t *partials = nullptr);

// W4A8 GEMM with per-block activation scales a_scale[m][k / block], block in
// {32, 64, 128}; out_dtype 0 (binary32) or 1 (bf16).
hipError_t launch_w4a8_gemm_blockact(const int8_t *a_q, const float *a_scale,
                                     const uint8_t *w_packed, const uint8_t *grp_scale,
                                     const float *ch_scale, int64_t m, int64_t n, int64_t k,
                                     int32_t block, void *out, int out_dtype,
                                     hipStream_t stream);

// EQuARX receive step: requantize(dequantize(q_in, s_in) + x) per block.
hipError_t launch_dequant_add_requant(const int8_t *q_in, const float *s_in, const void *x,
                                      bool x_bf16, int64_t rows, int64_t cols, int32_t block,
                                      float *sum_out, int8_t *q_out, float *s_out,
                                      hipStream_t stream);

// int8 matrix-core reference loop (measurement aid).
hipError_t launch_mfma_probe(int64_t workgroups, int32_t iters, int32_t *sink, uint64_t *clocks,
                             hipStream_t stream);

}  // namespace w4a8
