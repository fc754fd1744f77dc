// equarx.hip -- the local step of a block-quantized reduce-scatter for gfx950:
// dequantize a received int8 block to binary32, add the local partial sum, and
// quantize the result again, per block, in one pass over HBM.
//
// Method: "EQuARX" verdict page (pith.science arXiv 2506.17615),
// pith_extraction.key_machinery -- shards travel as block-wise symmetric int8
// with one binary32 scale per block; a receiver dequantizes each incoming
// block to FP32 before adding it to its partial sum, so the arithmetic on
// partial sums stays in FP32; the sum is quantized again (scales first, then
// data) for the next hop.  Per block:
//   d = fl(q_in * s_in);  v = fl(x + d)   (x binary32, or bf16 widened exactly)
//   amax = max |v|,  s = amax / 127,  inv = 127 / amax (0 if amax == 0),
//   q_out = rne(v * inv) in [-127, 127]  (same rounding as quantize_act_blockwise)
// and optionally v itself (the binary32 partial sum) is stored.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a8 {
namespace {

// Eight elements of lane vector i: d + x in binary32.
template <bool XBF16>
__device__ __forceinline__ void step_values(const u32x2 qv, float s, const void *x, int64_t i,
                                            float v[8]) {
    float xf[8];
    if constexpr (XBF16) {
        bf16x8_to_f32(__builtin_nontemporal_load((const u32x4 *)x + i), xf);
    } else {
        const f32x4 a = __builtin_nontemporal_load((const f32x4 *)x + 2 * i);
        const f32x4 b = __builtin_nontemporal_load((const f32x4 *)x + 2 * i + 1);
        xf[0] = a.x; xf[1] = a.y; xf[2] = a.z; xf[3] = a.w;
        xf[4] = b.x; xf[5] = b.y; xf[6] = b.z; xf[7] = b.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t w = e < 4 ? qv.x : qv.y;
        const int8_t c = (int8_t)((w >> (8 * (e & 3))) & 0xffu);
        const float d = (float)c * s;
        v[e] = xf[e] + d;
    }
}

__device__ __forceinline__ void store_sum(float *sum, int64_t i, const float v[8]) {
    f32x4 *o = (f32x4 *)sum;
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, &o[2 * i]);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, &o[2 * i + 1]);
}

// Blocks of 8 * LPB elements (LPB a power of two up to 64): the LPB lanes of a
// block are adjacent in a wavefront and reduce the maximum with shuffles.
template <int LPB, bool XBF16, bool SUM>
__global__ __launch_bounds__(256) void step_pow2_kernel(const u32x2 *__restrict__ q_in,
                                                        const float *__restrict__ s_in,
                                                        const void *__restrict__ x, int64_t nvec,
                                                        float *__restrict__ sum,
                                                        u32x2 *__restrict__ q_out,
                                                        float *__restrict__ s_out) {
    constexpr int U = 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += U * stride) {
        u32x2 qv[U];
        float sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = i + u * stride;
            if (idx < nvec) {
                qv[u] = __builtin_nontemporal_load(&q_in[idx]);
                sv[u] = s_in[idx / LPB];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = i + u * stride;
            // nvec is a multiple of LPB, so a block's lanes agree on this branch.
            if (idx < nvec) {
                float v[8];
                step_values<XBF16>(qv[u], sv[u], x, idx, v);
                float amax = absmax_f32x8(v);
#pragma unroll
                for (int off = 1; off < LPB; off <<= 1)
                    amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
                float s, inv;
                act_scale_pair(amax, s, inv);
                q_out[idx] = codes8(v, inv);
                if ((idx & (LPB - 1)) == 0) s_out[idx / LPB] = s;
                if constexpr (SUM) store_sum(sum, idx, v);
            }
        }
    }
}

// Any block that is a multiple of 8: one 256-thread workgroup per block; the
// block is read once for its maximum and again (from cache) for the codes.
template <bool XBF16, bool SUM>
__global__ __launch_bounds__(256) void step_wide_kernel(const u32x2 *__restrict__ q_in,
                                                        const float *__restrict__ s_in,
                                                        const void *__restrict__ x,
                                                        int64_t nblocks, int64_t block_vecs,
                                                        float *__restrict__ sum,
                                                        u32x2 *__restrict__ q_out,
                                                        float *__restrict__ s_out) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    for (int64_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
        const int64_t base = b * block_vecs;
        const float sb = s_in[b];
        float amax = 0.0f;
        for (int64_t j = tid; j < block_vecs; j += 256) {
            float v[8];
            step_values<XBF16>(q_in[base + j], sb, x, base + j, v);
            amax = __builtin_fmaxf(amax, absmax_f32x8(v));
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        __syncthreads();
        amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
        __syncthreads();
        float s, inv;
        act_scale_pair(amax, s, inv);
        for (int64_t j = tid; j < block_vecs; j += 256) {
            float v[8];
            step_values<XBF16>(q_in[base + j], sb, x, base + j, v);
            q_out[base + j] = codes8(v, inv);
            if constexpr (SUM) store_sum(sum, base + j, v);
        }
        if (tid == 0) s_out[b] = s;
    }
}

int step_grid(int64_t nvec) {
    int64_t blocks = (nvec + 2 * 256 - 1) / (2 * 256);
    const int64_t cap = 256 * 32;
    if (blocks > cap) blocks = cap;
    return (int)(blocks < 1 ? 1 : blocks);
}

template <bool XBF16, bool SUM>
hipError_t launch_step(const int8_t *q_in, const float *s_in, const void *x, int64_t rows,
                       int64_t cols, int32_t block, float *sum, int8_t *q_out, float *s_out,
                       hipStream_t stream) {
    const int64_t nvec = rows * cols / 8;
    const u32x2 *qi = (const u32x2 *)q_in;
    u32x2 *qo = (u32x2 *)q_out;
    const int g = step_grid(nvec);
#define W4A8_STEP_POW2(L) \
    step_pow2_kernel<L, XBF16, SUM><<<g, 256, 0, stream>>>(qi, s_in, x, nvec, sum, qo, s_out)
    switch (block) {
        case 8: W4A8_STEP_POW2(1); break;
        case 16: W4A8_STEP_POW2(2); break;
        case 32: W4A8_STEP_POW2(4); break;
        case 64: W4A8_STEP_POW2(8); break;
        case 128: W4A8_STEP_POW2(16); break;
        case 256: W4A8_STEP_POW2(32); break;
        case 512: W4A8_STEP_POW2(64); break;
        default: {
            const int64_t nblocks = rows * (cols / block);
            const int64_t grid = nblocks < 65536 ? nblocks : 65536;
            step_wide_kernel<XBF16, SUM><<<(int)grid, 256, 0, stream>>>(
                qi, s_in, x, nblocks, (int64_t)(block / 8), sum, qo, s_out);
        }
    }
#undef W4A8_STEP_POW2
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant_add_requant(const int8_t *q_in, const float *s_in, const void *x,
                                      bool x_bf16, int64_t rows, int64_t cols, int32_t block,
                                      float *sum_out, int8_t *q_out, float *s_out,
                                      hipStream_t stream) {
    if (rows * cols == 0) return hipSuccess;
    if (x_bf16)
        return sum_out ? launch_step<true, true>(q_in, s_in, x, rows, cols, block, sum_out,
                                                 q_out, s_out, stream)
                       : launch_step<true, false>(q_in, s_in, x, rows, cols, block, nullptr,
                                                  q_out, s_out, stream);
    return sum_out ? launch_step<false, true>(q_in, s_in, x, rows, cols, block, sum_out, q_out,
                                              s_out, stream)
                   : launch_step<false, false>(q_in, s_in, x, rows, cols, block, nullptr, q_out,
                                               s_out, stream);
}

}  // namespace w4a8
