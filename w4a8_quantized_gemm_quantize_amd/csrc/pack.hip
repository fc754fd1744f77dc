// pack.hip -- two-level 4-bit weight quantization and packing (layout V1), and
// its inverse, for gfx950.
//
// Method: "LiquidGEMM" verdict page (pith.science arXiv 2509.01229),
// referee_report.summary -- weights are first quantized to INT8 per channel,
// then to 4 bits with a per-group scale; skeptic_critique.load_bearing_attack
// -- that group scale is an integer; referee_report.major_comments[2] (paper
// section 4, Eq. 7) -- it is bounded by 16 thanks to a protective INT8 range.
// Symmetric instance used here: level 1 maps the channel's absmax to 112
// (= 7 * 16); level 2 takes s_g = max(1, ceil(m_g / 7)) over each group of 64
// and q = rne(W8 / s_g) in [-7, 7], stored as the nibble q + 8.
//
// The same kernel also writes LiquidGEMM's own asymmetric LQQ format (same
// page, pith_extraction.key_machinery and referee_report.major_comments[2]):
// level 1 with protective range 119, then per group of 64 the minimum `min` and
// the span max - min of the int8 codes, the integer scale s = nearest integer
// to span / 15 (at least 1; never a tie since 15 is odd, at most 16), codes
// u = rne((W8 - min) / s) clamped to 15, and the parameter s | (128 + min) << 8.
// And the int8 weights of the W8A8 comparison path: level 1 with range 127 and
// no second level, 16 bytes per lane and K step.
//
// One 256-thread workgroup packs one tile of 16 output channels: pass 1 reduces
// the 16 channel maxima, pass 2 gives each wavefront one 128-wide K chunk at a
// time; lane (c, kq) quantizes the 16 weights it owns per K step, the four lanes
// of a group exchange their extrema with cross-lane shuffles, and each lane
// writes its own record of the packed layout.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a8 {
namespace {

__device__ __forceinline__ float absmax_bf16x8(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[i] << 16)));
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w[i] & 0xffff0000u)));
    }
    return m;
}

template <int WF>
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ w, int64_t k,
                                                   uint8_t *__restrict__ w_packed,
                                                   uint8_t *__restrict__ grp_param,
                                                   float *__restrict__ ch_scale) {
    constexpr float kRange = WF == kW4Sym ? 112.0f : WF == kW4Lqq ? 119.0f : 127.0f;
    __shared__ float inv_lds[kNTile];
    const int64_t t = blockIdx.x;
    const int64_t n0 = t * kNTile;
    const int tid = threadIdx.x;

    // Pass 1: channel absmax c, ch_scale = c / range, inverse range / c.
    {
        const int r = tid >> 4, p = tid & 15;
        const uint4 *row = (const uint4 *)(w + (n0 + r) * k);
        float amax = 0.0f;
        for (int64_t v = p; v < k / 8; v += 16) amax = __builtin_fmaxf(amax, absmax_bf16x8(row[v]));
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
        if (p == 0) {
            ch_scale[n0 + r] = amax / kRange;
            inv_lds[r] = (amax > 0.0f) ? (kRange / amax) : 0.0f;
        }
    }
    __syncthreads();

    // Pass 2: one 128-wide chunk per wavefront.
    const int wave = tid >> 6, lane = tid & 63;
    const int c = lane & 15, kq = lane >> 4;
    const float inv = inv_lds[c];
    const int64_t nchunks = (k + kChunkK - 1) / kChunkK;
    const int64_t G = k / kGroup;
    const uint16_t *wrow = w + (n0 + c) * k;
    for (int64_t j = wave; j < nchunks; j += 4) {
        const bool full = (j + 1) * kChunkK <= k;
        uint32_t rec[4] = {0u, 0u, 0u, 0u};
        for (int h = 0; h < (full ? 2 : 1); ++h) {
            const int64_t k0 = j * kChunkK + h * kGroup + kq * 16;
            const uint4 v0 = *(const uint4 *)(wrow + k0);
            const uint4 v1 = *(const uint4 *)(wrow + k0 + 8);
            const uint32_t words[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            int w8[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                uint32_t bits = (e & 1) ? (words[e >> 1] & 0xffff0000u) : (words[e >> 1] << 16);
                w8[e] = sat_rne_code(__uint_as_float(bits) * inv, kRange);
            }
            const int64_t pidx = t * kNTile * G + (2 * j + h) * kNTile + c;
            uint32_t u[16];
            if constexpr (WF == kW8) {
                uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e) b[e >> 2] |= ((uint32_t)w8[e] & 0xffu) << (8 * (e & 3));
                *(uint4 *)(w_packed + wchunk_offset<kW8>(t, j, k) + h * kChunkBytes + lane * 16) =
                    make_uint4(b[0], b[1], b[2], b[3]);
                continue;
            } else if constexpr (WF == kW4Sym) {
                int m = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = max(m, abs(w8[e]));
                // the four lanes (kq = 0..3) holding one group of one channel
                m = max(m, __shfl_xor(m, 16));
                m = max(m, __shfl_xor(m, 32));
                const int s = (m == 0) ? 1 : (m + 6) / 7;
                const float fs = (float)s;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    // w8 / s is exact-rational; binary32 division then rint rounds it
                    // half to even because non-tie quotients sit >= 1/32 away from any
                    // half.
                    int qv = (int)__builtin_rintf((float)w8[e] / fs);
                    u[e] = (uint32_t)(qv + 8);
                }
                if (kq == 0) grp_param[pidx] = (uint8_t)s;
            } else {
                int lo = w8[0], hi = w8[0];
#pragma unroll
                for (int e = 1; e < 16; ++e) {
                    lo = min(lo, w8[e]);
                    hi = max(hi, w8[e]);
                }
                lo = min(lo, __shfl_xor(lo, 16));
                lo = min(lo, __shfl_xor(lo, 32));
                hi = max(hi, __shfl_xor(hi, 16));
                hi = max(hi, __shfl_xor(hi, 32));
                const int span = hi - lo;
                int s = span / 15 + ((span % 15) * 2 > 15 ? 1 : 0);
                s = s < 1 ? 1 : s;
                const float fs = (float)s;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    // (w8 - lo) / s in [0, 238]: the same exactness argument as above
                    int qv = (int)__builtin_rintf((float)(w8[e] - lo) / fs);
                    u[e] = (uint32_t)(qv < 15 ? qv : 15);
                }
                if (kq == 0)
                    ((uint16_t *)grp_param)[pidx] = (uint16_t)(s | ((128 + lo) << 8));
            }
            uint32_t p0 = 0u, p1 = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                p0 |= (u[b] | (u[4 + b] << 4)) << (8 * b);
                p1 |= (u[8 + b] | (u[12 + b] << 4)) << (8 * b);
            }
            rec[2 * h] = p0;
            rec[2 * h + 1] = p1;
        }
        if constexpr (WF != kW8) {
            uint8_t *dst = w_packed + packed_chunk_offset(t, j, k);
            if (full)
                *(uint4 *)(dst + lane * 16) = make_uint4(rec[0], rec[1], rec[2], rec[3]);
            else
                *(uint2 *)(dst + lane * 8) = make_uint2(rec[0], rec[1]);
        }
    }
}

// Inverse: one thread per (tile, chunk, lane) record.  Outputs in plain
// row-major order: codes q [n, k] (int8 q for kW4Sym and kW8, uint8 q_u4 for
// kW4Lqq), and for the 4-bit formats the group scale s [n, G] and, for kW4Lqq,
// the group minimum gmin [n, G].
template <int WF>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ w_packed,
                                                     const uint8_t *__restrict__ grp_param,
                                                     int64_t ntiles, int64_t k,
                                                     int8_t *__restrict__ q,
                                                     uint8_t *__restrict__ s_g,
                                                     int8_t *__restrict__ gmin) {
    const int64_t nchunks = (k + kChunkK - 1) / kChunkK;
    const int64_t G = k / kGroup;
    const int64_t total = ntiles * nchunks * 64;
    for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
         id += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(id & 63);
        const int64_t j = (id >> 6) % nchunks;
        const int64_t t = (id >> 6) / nchunks;
        const int c = lane & 15, kq = lane >> 4;
        const bool full = (j + 1) * kChunkK <= k;
        if constexpr (WF == kW8) {
            for (int h = 0; h < (full ? 2 : 1); ++h) {
                const uint8_t *src = w_packed + wchunk_offset<kW8>(t, j, k) + h * kChunkBytes +
                                     lane * 16;
                const int64_t n = t * kNTile + c;
                const int64_t k0 = j * kChunkK + h * kGroup + kq * 16;
                for (int e = 0; e < 16; ++e) q[n * k + k0 + e] = (int8_t)src[e];
            }
            continue;
        }
        const uint8_t *src = w_packed + packed_chunk_offset(t, j, k) + lane * (full ? 16 : 8);
        for (int h = 0; h < (full ? 2 : 1); ++h) {
            const uint32_t p[2] = {*(const uint32_t *)(src + 8 * h),
                                   *(const uint32_t *)(src + 8 * h + 4)};
            const int64_t g = 2 * j + h;
            const int64_t n = t * kNTile + c;
            const int64_t k0 = j * kChunkK + h * kGroup + kq * 16;
            for (int e = 0; e < 16; ++e) {
                const int d = e >> 2;
                const uint32_t u = (p[d >> 1] >> (8 * (e & 3) + 4 * (d & 1))) & 0xfu;
                q[n * k + k0 + e] = (int8_t)(WF == kW4Sym ? (int)u - 8 : (int)u);
            }
            if (kq == 0) {
                const int64_t pidx = t * kNTile * G + g * kNTile + c;
                if constexpr (WF == kW4Sym) {
                    s_g[n * G + g] = grp_param[pidx];
                } else {
                    const uint32_t v = ((const uint16_t *)grp_param)[pidx];
                    s_g[n * G + g] = (uint8_t)(v & 0xffu);
                    gmin[n * G + g] = (int8_t)((int)(v >> 8) - 128);
                }
            }
        }
    }
}

template <int WF>
hipError_t pack_fmt(const uint16_t *w, int64_t n, int64_t k, uint8_t *w_packed,
                    uint8_t *grp_param, float *ch_scale, hipStream_t stream) {
    const int64_t ntiles = n / kNTile;
    if (ntiles == 0) return hipSuccess;
    // k == 0 still runs: every channel maximum is 0, so ch_scale becomes 0.
    pack_kernel<WF><<<(unsigned)ntiles, 256, 0, stream>>>(w, k, w_packed, grp_param, ch_scale);
    return hipGetLastError();
}

template <int WF>
hipError_t unpack_fmt(const uint8_t *w_packed, const uint8_t *grp_param, int64_t n, int64_t k,
                      int8_t *q, uint8_t *s_g, int8_t *gmin, hipStream_t stream) {
    const int64_t ntiles = n / kNTile;
    if (ntiles == 0 || k == 0) return hipSuccess;
    const int64_t total = ntiles * ((k + kChunkK - 1) / kChunkK) * 64;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    unpack_kernel<WF><<<(unsigned)blocks, 256, 0, stream>>>(w_packed, grp_param, ntiles, k, q,
                                                            s_g, gmin);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_w4(const uint16_t *w, int64_t n, int64_t k, uint8_t *w_packed,
                          uint8_t *grp_scale, float *ch_scale, hipStream_t stream) {
    return pack_fmt<kW4Sym>(w, n, k, w_packed, grp_scale, ch_scale, stream);
}

hipError_t launch_unpack_w4(const uint8_t *w_packed, const uint8_t *grp_scale, int64_t n,
                            int64_t k, int8_t *q, uint8_t *s_g, hipStream_t stream) {
    return unpack_fmt<kW4Sym>(w_packed, grp_scale, n, k, q, s_g, nullptr, stream);
}

hipError_t launch_pack_w4_lqq(const uint16_t *w, int64_t n, int64_t k, uint8_t *w_packed,
                              uint16_t *grp_param, float *ch_scale, hipStream_t stream) {
    return pack_fmt<kW4Lqq>(w, n, k, w_packed, (uint8_t *)grp_param, ch_scale, stream);
}

hipError_t launch_unpack_w4_lqq(const uint8_t *w_packed, const uint16_t *grp_param, int64_t n,
                                int64_t k, uint8_t *q_u4, uint8_t *s_u8, int8_t *w_min,
                                hipStream_t stream) {
    return unpack_fmt<kW4Lqq>(w_packed, (const uint8_t *)grp_param, n, k, (int8_t *)q_u4, s_u8,
                              w_min, stream);
}

hipError_t launch_pack_w8(const uint16_t *w, int64_t n, int64_t k, int8_t *w_packed,
                          float *ch_scale, hipStream_t stream) {
    return pack_fmt<kW8>(w, n, k, (uint8_t *)w_packed, nullptr, ch_scale, stream);
}

hipError_t launch_unpack_w8(const int8_t *w_packed, int64_t n, int64_t k, int8_t *q8,
                            hipStream_t stream) {
    return unpack_fmt<kW8>((const uint8_t *)w_packed, nullptr, n, k, q8, nullptr, nullptr,
                           stream);
}

}  // namespace w4a8
