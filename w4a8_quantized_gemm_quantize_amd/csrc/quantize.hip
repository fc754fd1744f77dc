// quantize.hip -- block-wise absmax int8 quantization of bf16 activations and
// its dequantization, for gfx950.
//
// Method: "EQuARX" verdict page (pith.science arXiv 2506.17615),
// pith_extraction.key_machinery -- one binary32 scale per block from the
// block's absolute maximum (phase 1), then the data scaled and rounded to int8
// (phase 2); dequantization multiplies back to binary32.  Both phases run in
// one pass: each element is read from HBM once, kept in registers while the
// block maximum is reduced across lanes, then scaled and stored.
//
// Per block: s = amax / 127, inv = 127 / amax (0 when amax == 0),
// q = clamp(rne(x * inv), -127, 127), NaN products give 0.  Both divisions are
// correctly rounded binary32 divisions (HIP's default) and nothing is
// contracted (-ffp-contract=off), so codes and scales are exact functions of
// the bf16 input.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a8 {
namespace {

// Blocks of 8 * LPB elements (LPB = 1..64 lanes, a power of two).  The tensor
// is a flat sequence of blocks (cols % block == 0), so thread i owns the
// 16-byte vector i and the LPB lanes of one block are adjacent in a wavefront;
// the block maximum is a DPP reduction over those lanes.  The grid is a fixed
// 512 workgroups striding over the tensor, four vectors per lane per pass: on
// 64M elements that sweep reads and writes HBM faster than one workgroup per
// 1024 vectors (blocks 32 / 128: 38.2 -> 35.3 us / 38.1 -> 34.9 us, same box,
// interleaved).  The next pass's four vectors are requested before the
// current pass is converted, so eight are in flight per lane (64M elements,
// blocks 32 / 64 / 128: 39.2 -> 37.1, 39.7 -> 36.4, 37.2 -> 35.3 us, same box,
// two rotating buffer sets).
template <int LPB>
__global__ __launch_bounds__(256) void quant_pow2_kernel(const u32x4 *__restrict__ x,
                                                         int64_t nvec, u32x2 *__restrict__ q,
                                                         float *__restrict__ scales) {
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t step = U * stride;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nvec) return;
    // two register sets in turn: the next pass's vectors are requested before
    // this pass is converted and stored (clamped addresses past the end, never
    // used), so each lane keeps eight vectors in flight
    auto load = [&](u32x4 (&v)[U], int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * stride;
            v[u] = __builtin_nontemporal_load(&x[idx < nvec ? idx : nvec - 1]);
        }
    };
    auto work = [&](const u32x4 (&v)[U], int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t idx = base + u * stride;
            // nvec is a multiple of LPB, so a block's lanes agree on this branch.
            if (idx < nvec) {
                float f[8];
                bf16x8_to_f32(v[u], f);
                float amax = absmax_f32x8(f);
                amax = __uint_as_float(group_max_u32<LPB>(__float_as_uint(amax)));
                float s, inv;
                act_scale_pair(amax, s, inv);
                q[idx] = codes8(f, inv);
                if ((idx & (LPB - 1)) == 0) scales[idx / LPB] = s;
            }
        }
    };
    u32x4 a[U], b[U];
    load(a, i);
    while (true) {
        load(b, i + step);
        __builtin_amdgcn_sched_barrier(0);
        work(a, i);
        i += step;
        if (i >= nvec) break;
        load(a, i + step);
        __builtin_amdgcn_sched_barrier(0);
        work(b, i);
        i += step;
        if (i >= nvec) break;
    }
}

// Blocks of up to 64 * V vectors (8 elements each), one wavefront per block and
// four per workgroup: each lane holds V vectors, all requested before any is
// used (indices past the block are clamped to its last vector and ignored), so
// a lane has V loads in flight; the block maximum is a wavefront reduction with
// no barrier.  Per-token rows up to 8192 elements take this path.
template <int V>
__global__ __launch_bounds__(256) void quant_row_wave_kernel(const u32x4 *__restrict__ x,
                                                             int64_t nblocks, int block_vecs,
                                                             u32x2 *__restrict__ q,
                                                             float *__restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < nblocks; b += nwaves) {
        const u32x4 *xb = x + b * block_vecs;
        u32x4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int idx = lane + u * 64;
            v[u] = __builtin_nontemporal_load(xb + (idx < block_vecs ? idx : block_vecs - 1));
        }
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            float f[8];
            bf16x8_to_f32(v[u], f);
            if (lane + u * 64 < block_vecs) amax = __builtin_fmaxf(amax, absmax_f32x8(f));
        }
        // amax >= 0 and never NaN, so its bits order like unsigned integers
        amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
        float s, inv;
        act_scale_pair(amax, s, inv);
        u32x2 *qb = q + b * block_vecs;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int idx = lane + u * 64;
            if (idx < block_vecs) {
                float f[8];
                bf16x8_to_f32(v[u], f);
                __builtin_nontemporal_store(codes8(f, inv), qb + idx);
            }
        }
        if (lane == 0) scales[b] = s;
    }
}

// Longer blocks (any multiple of 8): one 256-thread workgroup per block.  Up to
// 256 * MAXV vectors stay in registers between the two phases, all requested
// before any is used (clamped indices, as above); a longer block is read a
// second time (from cache) for phase 2.
template <int MAXV>
__global__ __launch_bounds__(256) void quant_wide_kernel(const u32x4 *__restrict__ x,
                                                         int64_t nblocks, int64_t block_vecs,
                                                         u32x2 *__restrict__ q,
                                                         float *__restrict__ scales) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    for (int64_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
        const int64_t base = b * block_vecs;
        u32x4 v[MAXV];
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            const int64_t idx = tid + (int64_t)u * 256;
            v[u] = __builtin_nontemporal_load(&x[base + (idx < block_vecs ? idx : block_vecs - 1)]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            float f[8];
            bf16x8_to_f32(v[u], f);
            if (tid + (int64_t)u * 256 < block_vecs) amax = __builtin_fmaxf(amax, absmax_f32x8(f));
        }
        for (int64_t idx = tid + (int64_t)MAXV * 256; idx < block_vecs; idx += 256) {
            float f[8];
            bf16x8_to_f32(x[base + idx], f);
            amax = __builtin_fmaxf(amax, absmax_f32x8(f));
        }
        amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        __syncthreads();
        amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
        __syncthreads();
        float s, inv;
        act_scale_pair(amax, s, inv);
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            const int64_t idx = tid + (int64_t)u * 256;
            if (idx < block_vecs) {
                float f[8];
                bf16x8_to_f32(v[u], f);
                __builtin_nontemporal_store(codes8(f, inv), &q[base + idx]);
            }
        }
        for (int64_t idx = tid + (int64_t)MAXV * 256; idx < block_vecs; idx += 256) {
            float f[8];
            bf16x8_to_f32(x[base + idx], f);
            q[base + idx] = codes8(f, inv);
        }
        if (tid == 0) scales[b] = s;
    }
}

// Long blocks of up to 1024 * MAXV vectors (per-token rows of 8K-32K
// elements): one 1024-thread workgroup per block, striding over the blocks.
// All 16 wavefronts of a workgroup load at once, so even a short grid keeps
// enough loads in flight: 64 x 28672 took 4.3 us with a 256-thread workgroup
// per row and takes 3.2 us here; 2048 x 28672: 31.2 -> 29.7 us; 4096 x 16384:
// 40.6 -> 34.9 us.  The block maximum is a wavefront reduction, then one over
// the 16 wavefronts in LDS.
template <int MAXV>
__global__ __launch_bounds__(1024) void quant_wide1k_kernel(const u32x4 *__restrict__ x,
                                                            int64_t nblocks, int64_t block_vecs,
                                                            u32x2 *__restrict__ q,
                                                            float *__restrict__ scales) {
    __shared__ uint32_t red[16];
    const int tid = threadIdx.x;
    for (int64_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
        const int64_t base = b * block_vecs;
        u32x4 v[MAXV];
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            const int64_t idx = tid + (int64_t)u * 1024;
            v[u] = __builtin_nontemporal_load(&x[base + (idx < block_vecs ? idx : block_vecs - 1)]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            float f[8];
            bf16x8_to_f32(v[u], f);
            if (tid + (int64_t)u * 1024 < block_vecs) amax = __builtin_fmaxf(amax, absmax_f32x8(f));
        }
        // amax >= 0 and never NaN, so its bits order like unsigned integers
        const uint32_t wm = wave_max_u32(__float_as_uint(amax));
        if ((tid & 63) == 0) red[tid >> 6] = wm;
        __syncthreads();
        uint32_t m = red[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = max(m, red[i]);
        __syncthreads();
        float s, inv;
        act_scale_pair(__uint_as_float(m), s, inv);
#pragma unroll
        for (int u = 0; u < MAXV; ++u) {
            const int64_t idx = tid + (int64_t)u * 1024;
            if (idx < block_vecs) {
                float f[8];
                bf16x8_to_f32(v[u], f);
                __builtin_nontemporal_store(codes8(f, inv), &q[base + idx]);
            }
        }
        if (tid == 0) scales[b] = s;
    }
}

// out = q * s (binary32), optionally rounded to bf16.  Thread i owns 8 codes.
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const u32x2 *__restrict__ q,
                                                      const float *__restrict__ scales,
                                                      int64_t nvec, int64_t block_vecs,
                                                      void *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        u32x2 c = __builtin_nontemporal_load(&q[i]);
        float s = scales[i / block_vecs];
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t w = e < 4 ? c.x : c.y;
            int8_t b = (int8_t)((w >> (8 * (e & 3))) & 0xffu);
            f[e] = (float)b * s;
        }
        if (BF16) {
            u32x4 o;
            o.x = bf16x2_rne(f[0], f[1]);
            o.y = bf16x2_rne(f[2], f[3]);
            o.z = bf16x2_rne(f[4], f[5]);
            o.w = bf16x2_rne(f[6], f[7]);
            __builtin_nontemporal_store(o, &((u32x4 *)out)[i]);
        } else {
            f32x4 *o = (f32x4 *)out;
            __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, &o[2 * i]);
            __builtin_nontemporal_store(f32x4{f[4], f[5], f[6], f[7]}, &o[2 * i + 1]);
        }
    }
}

// 256-thread workgroups for work_items items, per_thread per thread, at most cap.
int grid_for(int64_t work_items, int per_thread, int64_t cap = 256 * 32) {
    int64_t threads = (work_items + per_thread - 1) / per_thread;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t *x, int64_t rows, int64_t cols, int32_t block,
                               int8_t *q, float *scales, hipStream_t stream) {
    const int64_t nvec = rows * cols / 8;
    const u32x4 *xv = (const u32x4 *)x;
    u32x2 *qv = (u32x2 *)q;
    if (nvec == 0) return hipSuccess;
    const int lpb = block / 8;
    const int g = grid_for(nvec, 4, 512);
    switch (block) {
        case 8: quant_pow2_kernel<1><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        case 16: quant_pow2_kernel<2><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        case 32: quant_pow2_kernel<4><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        case 64: quant_pow2_kernel<8><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        case 128: quant_pow2_kernel<16><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        case 256: quant_pow2_kernel<32><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        case 512: quant_pow2_kernel<64><<<g, 256, 0, stream>>>(xv, nvec, qv, scales); break;
        default: {
            const int64_t nblocks = rows * (cols / block);
            if (lpb <= 64 * 16) {
                // one wavefront per block, four per workgroup
                const int64_t wg = (nblocks + 3) / 4;
                const int grid = (int)(wg < 65536 ? wg : 65536);
                if (lpb <= 64)
                    quant_row_wave_kernel<1><<<grid, 256, 0, stream>>>(xv, nblocks, lpb, qv, scales);
                else if (lpb <= 128)
                    quant_row_wave_kernel<2><<<grid, 256, 0, stream>>>(xv, nblocks, lpb, qv, scales);
                else if (lpb <= 256)
                    quant_row_wave_kernel<4><<<grid, 256, 0, stream>>>(xv, nblocks, lpb, qv, scales);
                else if (lpb <= 512)
                    quant_row_wave_kernel<8><<<grid, 256, 0, stream>>>(xv, nblocks, lpb, qv, scales);
                else
                    quant_row_wave_kernel<16><<<grid, 256, 0, stream>>>(xv, nblocks, lpb, qv, scales);
            } else if (lpb <= 1024 * 4) {
                // blocks of up to 32768 elements: a 1024-thread workgroup each
                const int grid = (int)(nblocks < 65536 ? nblocks : 65536);
                quant_wide1k_kernel<4><<<grid, 1024, 0, stream>>>(xv, nblocks, (int64_t)lpb, qv,
                                                                 scales);
            } else {
                const int grid = (int)(nblocks < 65536 ? nblocks : 65536);
                quant_wide_kernel<16><<<grid, 256, 0, stream>>>(xv, nblocks, (int64_t)lpb, qv,
                                                                scales);
            }
        }
    }
    return hipGetLastError();
}

hipError_t launch_dequantize_act(const int8_t *q, const float *scales, int64_t rows,
                                 int64_t cols, int32_t block, void *out, bool bf16,
                                 hipStream_t stream) {
    const int64_t nvec = rows * cols / 8;
    if (nvec == 0) return hipSuccess;
    const int g = grid_for(nvec, 4);
    if (bf16)
        dequant_kernel<true><<<g, 256, 0, stream>>>((const u32x2 *)q, scales, nvec, block / 8,
                                                    out);
    else
        dequant_kernel<false><<<g, 256, 0, stream>>>((const u32x2 *)q, scales, nvec, block / 8,
                                                     out);
    return hipGetLastError();
}

}  // namespace w4a8
