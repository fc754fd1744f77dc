// gemm_kernels.hpp -- W4A8 GEMM kernels for gfx950: int8 activations x packed
// 4-bit weights, int8 MFMA with exact int32 accumulation, integer group scales
// folded into the int8 weight operand, binary32 / bf16 / int32 epilogue.  The
// kernels are templates over the weight format (device_common.hpp: symmetric
// 4-bit, LQQ 4-bit, or int8 for the W8A8 comparison path); gemm_w4.hip,
// gemm_lqq.hip and gemm_w8.hip instantiate one format each.
//
// Method: "LiquidGEMM" verdict page (pith.science arXiv 2509.01229),
// referee_report.summary -- 4-bit weights are rebuilt to INT8 inside the kernel
// and multiplied on the matrix units into INT32; pith_extraction.key_machinery
// -- the rebuild is (u * s + a) XOR 0x80, one multiply-add and one XOR per four
// weights (device_common.hpp: dequant4).  Because the group scale is a small
// integer it is folded into the operand (q * s in [-112, 112] is still int8),
// so acc = sum_g s_g * P_g comes out of the MFMA with no per-group work on the
// accumulators.  The same page's ImFP pipeline (pith_extraction.key_machinery:
// loading, dequantization and MMA overlap) is realised here with LDS double
// buffering (tiled kernel) and load batches issued ahead of use (skinny kernel).
//
// Operand roles on v_mfma_i32_16x16x64_i8: the rebuilt weights are operand A
// (16 channels x 64 k; lane (c, kq) = c + 16 kq holds channel c, k = 16 kq ..
// 16 kq + 15 -- exactly one record of the packed layout), the activations are
// operand B (64 k x 16 rows; lane (r, kq) holds row r and the same 16 k).  The
// result D[channel][row] arrives in lane (r, kq), element i = channel 4 kq + i:
// four consecutive output columns of one output row per lane, stored as one
// 8-byte (bf16) or 16-byte (fp32, int32) write.
//
// Kernels:
//   gemm_skinny_kernel  m <= 64 (decode shapes, HBM-bound).  One workgroup per
//                       NT 16-channel tiles; its wavefronts split K; packed
//                       weights stream from HBM into registers, the next batch
//                       of chunks requested before the current one is used.
//                       Partial sums meet in LDS with integer adds (exact in any
//                       order).  The FUSED form takes bf16 activations and
//                       quantizes them per row into LDS (same codes8 rounding
//                       as quantize_act_blockwise) while the first weight batch
//                       is in flight.
//   gemm_tiled_kernel   m > 64 (prefill shapes, MFMA-bound).  256 x 256 tile per
//                       workgroup of 16 wavefronts (64 x 64 each, four per
//                       SIMD); activations (direct global -> LDS loads) and
//                       rebuilt int8 weight operands in double-buffered LDS,
//                       one K chunk (128) per barrier; each 16-channel weight
//                       tile is rebuilt once per workgroup, by one wavefront.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace w4a8 {
namespace {

// Workgroup barrier that waits only for this wavefront's LDS operations
// (lgkmcnt(0)): global loads stay in flight across it, so weight batches
// requested before it keep streaming in.  (__syncthreads() would wait for every
// outstanding load.)  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Epilogue for channels n..n+3 of output row `row` (n % 4 == 0).
__device__ __forceinline__ void store4(void *out, int out_dtype, int64_t row, int64_t ldo,
                                       int64_t n, v4i acc, float sa, f32x4 sc) {
    const int64_t idx = row * ldo + n;
    if (out_dtype == 2) {
        *(v4i *)((int *)out + idx) = acc;
        return;
    }
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        y[i] = (float)acc[i] * sa;
        y[i] = y[i] * sc[i];
    }
    if (out_dtype == 1) {
        const u32x2 b = {bf16x2_rne(y[0], y[1]),
                         bf16x2_rne(y[2], y[3])};
        *(u32x2 *)((uint16_t *)out + idx) = b;
    } else {
        *(f32x4 *)((float *)out + idx) = f32x4{y[0], y[1], y[2], y[3]};
    }
}

// Per-block activation scales (AB > 0): the int32 partial t of one activation
// block is folded into the binary32 accumulator as f = fl(fl(t) * s + f), one
// fused multiply-add (one rounding), block after block in K order.  |t| < 2^24,
// so fl(t) is exact.  The fold is VALU work on every output of every block
// (a conversion and an FMA); with the product and the sum rounded separately
// it was a third more (prefill 4096 x 14336 x 4096, block 128: 441 -> 407 us).
__device__ __forceinline__ void fold4(f32x4 &f, const v4i t, float s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __builtin_fmaf((float)t[i], s, f[i]);
}

// Epilogue of the per-block form: out = f * ch_scale, binary32 or bf16.
__device__ __forceinline__ void store4f(void *out, int out_dtype, int64_t row, int64_t ldo,
                                        int64_t n, f32x4 f, f32x4 sc) {
    const int64_t idx = row * ldo + n;
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = f[i] * sc[i];
    if (out_dtype == 1) {
        const u32x2 b = {bf16x2_rne(y[0], y[1]),
                         bf16x2_rne(y[2], y[3])};
        *(u32x2 *)((uint16_t *)out + idx) = b;
    } else {
        *(f32x4 *)((float *)out + idx) = f32x4{y[0], y[1], y[2], y[3]};
    }
}

// Activation operand restricted to one 32-wide half of a 64-wide K step: lanes
// kq = 0, 1 hold k 0..31 of the step, lanes kq = 2, 3 hold k 32..63.
__device__ __forceinline__ v4i half_operand(v4i a, int kq, int half) {
    return ((kq >> 1) == half) ? a : v4i{0, 0, 0, 0};
}

// Weight records streamed once from HBM: 16-byte buffer load with the
// nontemporal cache policy (cache policy operand 2), as the flat loads of the
// previous form had (__builtin_nontemporal_load); without it the decode
// kernels ran 2-7 % slower.
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
}

// ---------------------------------------------------------------- skinny --
constexpr int kSkinnyMaxVec = 8;    // fused prologue: 16-byte vectors held per thread
// Row vectors (8 activations each) per thread of the fused prologue with
// `waves` wavefronts: the rows split over threads in power-of-two groups.
inline int64_t fused_need(int64_t m, int64_t k, int waves) {
    const int64_t threads = 64 * waves;
    int64_t tpr = threads;
    while (tpr * m > threads) tpr >>= 1;
    return (k / 8 + tpr - 1) / tpr;
}
// Wavefronts per workgroup of the fused form.  8, with deeper load batches,
// once each wavefront's share of the weight stream is long enough (k > 2048);
// 16 for short rows (the prologue, which every workgroup runs over all of A,
// then dominates and gets four wavefronts per SIMD), when 8 wavefronts would
// need more than kSkinnyMaxVec vectors per thread, and when the workgroups
// fit one per CU with more than four vectors per thread (8 x 4096 x 4096:
// 6.50 us with 16, 6.86 with 8).  A/B on MI355X, fused calls, 16 -> 8
// wavefronts: 1 x 28672 x 4096 21.3 -> 15.9 us, 1 x 28672 x 8192 29.8 ->
// 24.8, 2 x 14336 x 4096 12.9 -> 10.4, 1 x 8192 x 8192 10.6 -> 9.7; at k =
// 2048 no difference.
constexpr int64_t kFusedShortK = 2048;
inline int fused_waves(int64_t m, int64_t n, int64_t k, int64_t ncu) {
    if (k <= kFusedShortK) return 16;
    const int64_t need8 = fused_need(m, k, 8);
    if (need8 > kSkinnyMaxVec) return 16;
    if (need8 > 4 && n / kNTile <= ncu) return 16;
    return 8;
}
// The 8-wavefront form with 4 vectors per thread takes two 16-channel tiles
// per workgroup (load batches of two chunks) when the grid would have more
// than two workgroups per CU and each converts at least 8192 activations:
// half the workgroups then repeat the conversion of A (A/B on MI355X, fused
// calls: 2 x 14336 x 4096 10.9 -> 9.8 us, 1 x 14336 x 8192 14.8 -> 13.4,
// 4 x 28672 x 4096 19.8 -> 18.6, 1 x 28672 x 8192 26.3 -> 24.8; with 4096
// activations no gain: 1 x 28672 x 4096 16.6 -> 16.8).
inline bool fused_two_tiles(int64_t m, int64_t n, int64_t k, int64_t ncu) {
    return n / kNTile > 2 * ncu && m * k >= 8192;
}

template <int WF, int NT, int D, int MT, bool WITH_ACT, int AB>
struct WeightBatch {
    WRec<WF> w[D][NT];                    // one packed record per chunk and tile
    uint32_t s[D][NT][2];                 // group parameters of the chunk's two K steps
    v4i a[WITH_ACT ? D : 1][2][MT];       // int8 activation fragments (non-fused)
    // per-block activation scales of the chunk's K steps (AB > 0): one or two
    // blocks per step and row tile, for this lane's row
    float sa[AB ? D : 1][2][AB ? MT : 1][AB == 32 ? 2 : 1];
};

// AV: 16-byte activation vectors per thread in the fused prologue (unused otherwise).
// AB: 0 = per-token activation scales a_scale[m]; 32, 64 or 128 = per-block
// scales a_scale[m][k / AB] folded per block (non-fused form only).
// KF: the fused prologue keeps the widened activations in registers between its
// maximum and its codes (fewer VALU instructions, more registers: used when one
// workgroup per CU is all the grid has, so occupancy does not matter).
template <int WF, int MT, int NT, int WAVES, int D, bool FUSED, int AV, int AB = 0,
          bool KF = false>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_kernel(
    const void *__restrict__ act, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ w_packed, const uint8_t *__restrict__ grp_scale,
    const float *__restrict__ ch_scale, int m, int64_t n, int64_t k,
    void *__restrict__ out, int out_dtype, int8_t *__restrict__ ws_q,
    float *__restrict__ ws_s, int64_t first_wave) {
    constexpr int THREADS = 64 * WAVES;
    constexpr int ROWS = MT * 16;
    extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];  // FUSED: [m][k + 16]
    static_assert(AB == 0 || !FUSED, "per-block scales only in the non-fused form");
    __shared__ int red[AB ? 1 : NT][16][AB ? 1 : ROWS + 4];
    __shared__ float redf[AB ? WAVES : 1][AB ? NT : 1][16][AB ? ROWS + 1 : 1];
    __shared__ float sa_lds[ROWS];
    __shared__ unsigned amax_lds[ROWS];

    const int tid = threadIdx.x;
    // readfirstlane: the compiler then knows the wavefront index, and so each
    // wavefront's chunk range and loop control, is uniform (scalar branches).
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, kq = lane >> 4;
    const int64_t ntiles = n / kNTile;
    const int64_t t0 = (int64_t)blockIdx.x * NT;
    // k <= K_MAX: the K-derived counts fit 32 bits (shorter scalar code ahead
    // of the first loads: 150 -> 123 instructions before the decode kernel's
    // last prologue request, decode 6.52 -> 6.46 us, 4 x 4096 x 4096 5.67 ->
    // 5.52 us on one box)
    const int k32 = (int)k;
    const int nchunks = (k32 + kChunkK - 1) >> 7;
    const int G = k32 >> 6;
    const int lds_stride = k32 + 16;

    if constexpr (AB == 0)
        for (int i = tid; i < NT * 16 * (ROWS + 4); i += THREADS) (&red[0][0][0])[i] = 0;
    const int64_t nblk = AB ? k / AB : 1;
    if (tid < ROWS) amax_lds[tid] = 0u;

    // Full 128-wide chunks are split evenly over the wavefronts; a trailing
    // 64-wide chunk (k % 128 == 64) is done by the last wavefront afterwards, so
    // the batched loads below carry no data-dependent branches.  The launchers
    // only use this kernel for k >= 128 (at least one full chunk), so a
    // wavefront without chunks of its own (j0 >= j1) still loads a valid one,
    // chunk j1 - 1 = nfull - 1, and never uses it.
    const int nfull = k32 >> 7;
    const bool has_half = nfull < nchunks;
    const int per = (nfull + WAVES - 1) / WAVES;
    const int j0 = wave * per;
    const int j1 = (j0 + per < nfull) ? j0 + per : nfull;
    const int8_t *a_q = (const int8_t *)act;

    // Buffer resources over this workgroup's weight tiles and their group
    // parameters (tiles past n read zero: they only reach unstored outputs)
    // and, without the fused prologue, over the m rows of activation codes.
    // Per-lane offsets are fixed for the whole K loop and the chunk goes in
    // the scalar offset, so the loads need no vector address arithmetic.  The
    // group parameter comes as the aligned 32-bit word that holds it and the
    // rebuild constants are taken out of it with one v_perm_b32 and one
    // v_pk_mad_u16 (device_common.hpp: wparam_consts).  All offsets fit 32
    // bits: k <= K_MAX, m <= 64.
    constexpr int kWTileMul = WF == kW8 ? 16 : 8;                // weight bytes per tile = mul * k
    constexpr int kPSize = WF == kW4Lqq ? 2 : 1;                 // bytes per group parameter
    const int wtile = kWTileMul * (int)k;
    const int ptile = kNTile * (int)G * kPSize;
    const int tiles_here = (int)(ntiles - t0 < NT ? ntiles - t0 : NT);
    const __amdgpu_buffer_rsrc_t rw =
        buffer_rsrc(w_packed + t0 * (int64_t)wtile, (uint32_t)tiles_here * wtile);
    const __amdgpu_buffer_rsrc_t rp =
        WF == kW8 ? rw : buffer_rsrc(grp_scale + t0 * (int64_t)ptile, (uint32_t)tiles_here * ptile);
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(act, FUSED ? (uint32_t)(m * k32 * 2) : (uint32_t)(m * k));
    const WParamSel psel = wparam_selectors<WF>(c);
    const int poff_c = WF == kW4Lqq ? (c & ~1) * 2 : (c & ~3);
    int aoff[FUSED ? 1 : MT];                    // activation row offsets (rows past m: row m - 1)
#pragma unroll
    for (int mt = 0; mt < (FUSED ? 1 : MT); ++mt) {
        const int row = (mt * 16 + c < m) ? mt * 16 + c : m - 1;
        aoff[mt] = row * (int)k + kq * 16;
    }

    // Weights (+ non-fused activation fragments) of D chunks, requested together.
    // Every load is unconditional: chunks past the wavefront's range and rows
    // past m are clamped to valid ones, tiles past n read zero, and nothing
    // they fetch is stored (chunks are skipped, those rows and tiles are not
    // stored).  A branch around a load would make the compiler wait for it at
    // the join.
    const int64_t tlast = ntiles - 1;
    auto load_batch = [&](WeightBatch<WF, NT, D, MT, !FUSED, AB> &b, int jb) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = (jb + d < j1) ? jb + d : j1 - 1;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (WF == kW8) {
                    b.w[d][nt].r0 = buffer_load16_nt(rw, nt * wtile + lane * 16, j * (2 * kChunkBytes));
                    b.w[d][nt].r1 = buffer_load16_nt(rw, nt * wtile + lane * 16,
                                                  j * (2 * kChunkBytes) + kChunkBytes);
                    b.s[d][nt][0] = b.s[d][nt][1] = 0u;
                } else {
                    b.w[d][nt].r = buffer_load16_nt(rw, nt * wtile + lane * 16, j * kChunkBytes);
                    const int so = j * (2 * kNTile * kPSize);
                    b.s[d][nt][0] = buffer_load4(rp, nt * ptile + poff_c, so);
                    b.s[d][nt][1] = buffer_load4(rp, nt * ptile + poff_c, so + kNTile * kPSize);
                }
            }
            if constexpr (!FUSED) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int row = (mt * 16 + c < m) ? mt * 16 + c : m - 1;
                        b.a[d][h][mt] = __builtin_bit_cast(
                            v4i, buffer_load16(ra, aoff[mt], j * kChunkK + h * kGroup));
                        if constexpr (AB > 0) {
                            const int64_t ks = 2 * j + h;                  // 64-wide K step
#pragma unroll
                            for (int sub = 0; sub < (AB == 32 ? 2 : 1); ++sub) {
                                const int64_t blk = AB == 32 ? 2 * ks + sub : AB == 64 ? ks : ks / 2;
                                b.sa[d][h][mt][sub] = a_scale[(int64_t)row * nblk + blk];
                            }
                        }
                    }
            }
        }
    };

    WeightBatch<WF, NT, D, MT, !FUSED, AB> cur;
    if constexpr (!FUSED) {
        load_batch(cur, j0);
        lds_barrier();  // red cleared
    } else {
        // Per-row absmax -> scale, then the row's codes into LDS.  Threads are
        // split into m groups of tpr (a power of two) threads per row.  All
        // loads are issued before any is used.
        const int vpr = k32 >> 3;
        int tpr = THREADS;
        while (tpr * m > THREADS) tpr >>= 1;
        const int row = tid / tpr, sub = tid % tpr;
        const bool row_ok = row < m;
        // Unconditional loads from clamped (valid) addresses; vectors outside the
        // row are ignored below.  32-bit buffer offsets (m k <= 16 K_MAX).
        const int rowbase = (row_ok ? row : m - 1) * vpr;
        u32x4 av[AV];
#pragma unroll
        for (int u = 0; u < AV; ++u) {
            const int v = sub + u * tpr;
            av[u] = buffer_load16(ra, (rowbase + (v < vpr ? v : vpr - 1)) * 16, 0);
        }
        // The first weight batch is requested after the activations: loads
        // complete in order, so waiting for the activations below does not wait
        // for the weights, which stream in while the prologue runs.  The
        // scheduling barrier keeps every activation load ahead of the weight
        // requests: the compiler had moved the last two of eight after the
        // group-parameter loads, and the row maximum then waited for those.
        __builtin_amdgcn_sched_barrier(0);
        load_batch(cur, j0);
        lds_barrier();  // red / amax_lds cleared
        // With KF each vector is widened once and the floats are kept for the
        // codes below.  When the row splits evenly over its threads (every
        // vector valid) the per-vector range checks are skipped.
        const bool all_valid = KF && row_ok && tpr * AV == vpr;
        float fa[KF ? AV : 1][8];
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < AV; ++u) {
            float f[8];
            bf16x8_to_f32(av[u], f);
            const float mx = absmax_f32x8(f);
            if constexpr (KF) {
#pragma unroll
                for (int i = 0; i < 8; ++i) fa[u][i] = f[i];
            }
            if (all_valid || (row_ok && sub + (int64_t)u * tpr < vpr))
                amax = __builtin_fmaxf(amax, mx);
        }
        // amax >= 0 and never NaN, so its bits order like unsigned integers.
        float inv;
        if (tpr == 64) {
            // One wavefront per row: reduce in registers, no barrier needed.
            const float rmax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
            float s;
            act_scale_pair(rmax, s, inv);
            if (row_ok && lane == 0) {
                sa_lds[row] = s;
                if (blockIdx.x == 0) ws_s[row] = s;
            }
        } else {
            // Rows spread over several wavefronts (tpr > 64) or share one (tpr < 64).
            if (tpr > 64) {
                const uint32_t wm = wave_max_u32(__float_as_uint(amax));
                if (row_ok && lane == 0) atomicMax(&amax_lds[row], wm);
            } else {
                for (int off = 1; off < tpr; off <<= 1)
                    amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
                if (row_ok && sub == 0) atomicMax(&amax_lds[row], __float_as_uint(amax));
            }
            lds_barrier();
            float s;
            act_scale_pair(__uint_as_float(amax_lds[row_ok ? row : 0]), s, inv);
            if (row_ok && sub == 0) {
                sa_lds[row] = s;
                if (blockIdx.x == 0) ws_s[row] = s;
            }
        }
        if (row_ok) {
#pragma unroll
            for (int u = 0; u < AV; ++u) {
                const int64_t v = sub + (int64_t)u * tpr;
                if (all_valid || v < vpr) {
                    float f[8];
                    if constexpr (KF) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) f[i] = fa[u][i];
                    } else {
                        bf16x8_to_f32(av[u], f);
                    }
                    const u32x2 q = codes8(f, inv);
                    *(u32x2 *)(act_lds + row * lds_stride + v * 8) = q;
                    if (blockIdx.x == 0) *(u32x2 *)(ws_q + row * k + v * 8) = q;
                }
            }
        }
        lds_barrier();
    }

    v4i acc[NT][MT];
    f32x4 accf[AB ? NT : 1][AB ? MT : 1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[nt][mt] = v4i{0, 0, 0, 0};
            if constexpr (AB > 0) accf[nt][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }

    // One K step (64) of one chunk: rebuild the weight operand of each tile and
    // multiply it into every row tile.  With per-block scales (sa: this lane's
    // row scales of the step's block(s)) each block's partial is folded as
    // soon as it is complete: per step for blocks of 32 (two half-step
    // products) and 64, every second step for 128.
    using SaStep = float[AB ? MT : 1][AB == 32 ? 2 : 1];
    auto mma_step = [&](const WRec<WF> rec[NT], int h, const uint32_t sv[NT],
                        const v4i av[MT], const SaStep &sa) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t mul = 0u, add = 0u;
            if constexpr (WF != kW8) wparam_consts<WF>(sv[nt], psel, mul, add);
            const v4i wv = wrec_operand_ma<WF>(rec[nt], h, mul, add);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (AB == 0) {
                    acc[nt][mt] = mfma16x16x64(wv, av[mt], acc[nt][mt]);
                } else if constexpr (AB == 32) {
                    const v4i zero = {0, 0, 0, 0};
                    fold4(accf[nt][mt], mfma16x16x64(wv, half_operand(av[mt], kq, 0), zero),
                          sa[mt][0]);
                    fold4(accf[nt][mt], mfma16x16x64(wv, half_operand(av[mt], kq, 1), zero),
                          sa[mt][AB == 32 ? 1 : 0]);
                } else if constexpr (AB == 64) {
                    fold4(accf[nt][mt], mfma16x16x64(wv, av[mt], v4i{0, 0, 0, 0}), sa[mt][0]);
                } else {
                    acc[nt][mt] = mfma16x16x64(wv, av[mt], acc[nt][mt]);
                    if (h == 1) {
                        fold4(accf[nt][mt], acc[nt][mt], sa[mt][0]);
                        acc[nt][mt] = v4i{0, 0, 0, 0};
                    }
                }
            }
        }
    };
    SaStep sa_none = {};
    // Activation fragments of rows mt * 16 + c; rows past m read row m - 1.
    // Their products land in accumulator rows that are never stored (the
    // reduction below stores rows < m only), so they need no masking.
    auto lds_act = [&](v4i av[MT], int64_t kk) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = (mt * 16 + c < m) ? mt * 16 + c : m - 1;
            av[mt] = *(const v4i *)(act_lds + row * lds_stride + kk);
        }
    };

    // The chunks of batch b starting at jb (the first `cnt` of its D are used).
    auto compute_batch = [&](const WeightBatch<WF, NT, D, MT, !FUSED, AB> &b, int jb, int cnt) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d >= cnt) break;
            const int j = jb + d;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t sv[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) sv[nt] = b.s[d][nt][h];
                v4i av[MT];
                if constexpr (FUSED) {
                    lds_act(av, j * kChunkK + h * kGroup + kq * 16);
                } else {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) av[mt] = b.a[d][h][mt];
                }
                if constexpr (AB > 0) mma_step(b.w[d], h, sv, av, b.sa[d][h]);
                else mma_step(b.w[d], h, sv, av, sa_none);
            }
        }
    };
    // Software pipeline over batches with two register sets used in turn: the
    // next batch is requested into the other set before the current one is
    // used, so multiplying a batch waits only for its own loads while the next
    // batch stays in flight (a copy from one set to the other would wait for
    // both).  The scheduling barriers keep the requests ahead of the uses:
    // the scheduler would otherwise sink them to reuse registers, exposing
    // their latency.
    //   With more workgroups than CUs, two share a CU and the issue arbiter
    // favours the older one's wavefronts; the two take turns at a raised
    // wave priority, batch by batch, so they stream their weights together
    // rather than one after the other (same boxes, interleaved: ffn-down
    // M = 16 41.5 -> 39.5 us, M = 1 22.8 -> 22.6 us; one workgroup per CU
    // unchanged).
    WeightBatch<WF, NT, D, MT, !FUSED, AB> other;
    int jb = j0;
    const bool second = (int64_t)blockIdx.x >= first_wave;
    while (true) {
        if (jb + D >= j1) {
            if (jb < j1) compute_batch(cur, jb, j1 - jb);
            break;
        }
        if (second) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        load_batch(other, jb + D);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch(cur, jb, D);
        jb += D;
        if (jb + D >= j1) {
            compute_batch(other, jb, j1 - jb);
            break;
        }
        if (second) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(1);
        load_batch(cur, jb + D);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch(other, jb, D);
        jb += D;
    }
    __builtin_amdgcn_s_setprio(0);

    if (has_half && wave == WAVES - 1) {
        // Trailing 64-wide chunk: one K step.
        const int64_t j = nfull;
        WRec<WF> wp[NT];
        uint32_t sv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int64_t t = (t0 + nt < ntiles) ? t0 + nt : tlast;
            wp[nt] = load_wrec_half<WF>(w_packed, t, j, k, lane);
            sv[nt] = WF == kW8 ? 0u
                               : buffer_load4(rp, nt * ptile + poff_c,
                                              (int)(2 * j) * kNTile * kPSize);
        }
        v4i av[MT];
        const int64_t kk = j * kChunkK + kq * 16;
        if constexpr (FUSED) {
            lds_act(av, kk);
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = (mt * 16 + c < m) ? mt * 16 + c : m - 1;
                av[mt] = *(const v4i *)(a_q + (int64_t)row * k + kk);
            }
        }
        SaStep sa_half = {};
        if constexpr (AB > 0) {
            // blocks of 32 or 64 only: k % 128 == 64 excludes blocks of 128
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = (mt * 16 + c < m) ? mt * 16 + c : m - 1;
#pragma unroll
                for (int sub = 0; sub < (AB == 32 ? 2 : 1); ++sub)
                    sa_half[mt][sub] =
                        a_scale[(int64_t)row * nblk + (AB == 32 ? 4 * j + sub : 2 * j)];
            }
        }
        mma_step(wp, 0, sv, av, sa_half);
    }

    if constexpr (AB > 0) {
        // binary32 partials of each wavefront; summed below in wavefront order
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) redf[wave][nt][4 * kq + i][mt * 16 + c] = accf[nt][mt][i];
        __syncthreads();
        for (int idx = tid; idx < NT * m * 4; idx += THREADS) {
            const int nt = idx / (m * 4);
            const int rem = idx - nt * m * 4;
            const int row = rem >> 2, quad = rem & 3;
            const int64_t t = t0 + nt;
            if (t >= ntiles) continue;
            f32x4 f = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int w = 0; w < WAVES; ++w)
#pragma unroll
                for (int i = 0; i < 4; ++i) f[i] = f[i] + redf[w][nt][4 * quad + i][row];
            const int64_t nn = t * kNTile + 4 * quad;
            store4f(out, out_dtype, row, n, nn, f, *(const f32x4 *)(ch_scale + nn));
        }
        return;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(&red[nt][4 * kq + i][mt * 16 + c], acc[nt][mt][i]);
    __syncthreads();
    for (int idx = tid; idx < NT * m * 4; idx += THREADS) {
        const int nt = idx / (m * 4);
        const int rem = idx - nt * m * 4;
        const int row = rem >> 2, quad = rem & 3;
        const int64_t t = t0 + nt;
        if (t >= ntiles) continue;
        const v4i a4 = {red[nt][4 * quad][row], red[nt][4 * quad + 1][row],
                        red[nt][4 * quad + 2][row], red[nt][4 * quad + 3][row]};
        const int64_t nn = t * kNTile + 4 * quad;
        const float sa = FUSED ? sa_lds[row] : a_scale[row];
        store4(out, out_dtype, row, n, nn, a4, sa, *(const f32x4 *)(ch_scale + nn));
    }
}

// ----------------------------------------------------------------- tiled --
// BM x BN output tile per workgroup of WAVES_M x WAVES_N wavefronts, each
// wavefront (BM / WAVES_M) x (BN / WAVES_N).  K advances one 128-wide chunk per
// barrier through two LDS stages, each holding
//   act: [BM][128] int8 activations (16-byte columns XOR-swizzled by row % 8),
//   w:   [BN/16][2 steps][64 lanes][16 B] rebuilt int8 weight operands, each
//        exactly the operand A of v_mfma_i32_16x16x64_i8 for 16 channels.
// Weights are rebuilt once per workgroup, not once per wavefront: while the
// workgroup multiplies chunk j, each wavefront fetches the packed records of
// its own 16-channel tile(s) for chunk j + 1 straight into registers, rebuilds
// them (unpack + group scale, device_common.hpp) and writes the int8 operands
// into the other stage.  The MFMA loop itself is LDS reads and MFMAs only, and
// small per-wavefront register budgets keep four wavefronts per SIMD so the
// matrix cores always have work to issue.
// With one row of wavefronts (WAVES_M == 1) each wavefront multiplies only the
// tiles it fetches, so the weight stage is skipped: operands are rebuilt in
// registers right before their MFMAs, and three activation stages keep two
// chunks of loads in flight (the split-K tile and the tail launch).
template <int BM, int BN>
struct TiledLds {
    static constexpr int kAct = BM * kChunkK;                 // activations
    static constexpr int kW = (BN / 16) * 2 * kChunkBytes;     // rebuilt weights
};

// Byte offset of 16-byte column c16 (0..7) of activation row `row` in LDS.  The
// 16 x 16 x 64 MFMA operand read has 16 consecutive rows at one column per
// 16-lane group; XOR-ing the column with row % 8 makes that ds_read_b128
// conflict-free on gfx950 (measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int act_swz(int row, int c16) { return c16 ^ (row & 7); }
__device__ __forceinline__ int act_lds_off(int row, int c16) {
    return row * kChunkK + (act_swz(row, c16) << 4);
}

// AB: 0 = per-token activation scales; 32, 64 or 128 = per-block scales
// a_scale[m][k / AB], each block's int32 partial folded into binary32 in K order.
// kslice (a multiple of 128): blockIdx.y = s takes K range [s kslice, (s + 1)
// kslice) and writes its int32 partial sums (out_dtype 2) to slice s of `out`,
// [gridDim.y][m][ldo]; one slice (kslice >= k) is the whole product.  Per-token
// scales only when split.  first_wave: workgroups the device starts before the
// rest (one per CU); with two per CU the later one of each pair is second.
template <int WF, int BM, int BN, int WAVES_M, int WAVES_N, int AB = 0>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, AB == 64 || AB == 128 ? 2 : 1) void gemm_tiled_kernel(
    const int8_t *__restrict__ a_q, const float *__restrict__ a_scale,
    const uint8_t *__restrict__ w_packed, const uint8_t *__restrict__ grp_scale,
    const float *__restrict__ ch_scale, int64_t m, int64_t n, int64_t k,
    void *__restrict__ out, int64_t ldo, int out_dtype, int64_t kslice, int64_t first_wave) {
    using L = TiledLds<BM, BN>;
    constexpr int WAVES = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;   // 16 x 16 MFMA tiles per wavefront
    constexpr int NTB = BN / 16;              // 16-channel tiles per workgroup
    constexpr int TPW = NTB / WAVES;          // tiles each wavefront rebuilds
    constexpr int ACT_I = BM / 8 / WAVES;     // 1 KB activation blocks per wavefront
    static_assert(TPW >= 1 && TPW * WAVES == NTB, "one or more weight tiles per wavefront");
    static_assert(ACT_I >= 1 && ACT_I * WAVES * 8 == BM, "activation blocks per wavefront");
    // With the wavefronts side by side in N (WAVES_M == 1) a wavefront consumes
    // exactly the tiles whose records it fetches (TPW == TN).  Its weight
    // operands are then rebuilt in registers right before their MFMAs and never
    // pass through LDS (LDS writes are the slow side of LDS on gfx950); each
    // tile is still rebuilt once per workgroup.
    constexpr bool kRegW = WAVES_M == 1 && TPW == TN;
    // Each stage of each operand is its own array and the chunk loop is unrolled
    // by two so every access names its array statically: the direct-to-LDS
    // activation loads into one stage then provably never alias reads of the
    // other stage or the weight writes, and the compiler does not make those
    // wait for the loads in flight.
    __shared__ __attribute__((aligned(16))) uint8_t act0[L::kAct];
    __shared__ __attribute__((aligned(16))) uint8_t act1[L::kAct];
    // kRegW: a third activation stage (the K loop runs two chunks ahead), and
    // the weight arrays only stage the epilogue (half the wavefronts each).
    constexpr int kEpiW = (WAVES / 2) * WM * WN * 2;
    __shared__ __attribute__((aligned(16))) uint8_t act2[kRegW ? L::kAct : 16];
    __shared__ __attribute__((aligned(16))) uint8_t wl0[kRegW ? kEpiW : L::kW];
    __shared__ __attribute__((aligned(16))) uint8_t wl1[kRegW ? kEpiW : L::kW];
    // Per-token scales of the tile's rows and channel scales of its columns,
    // whole 1 KB blocks for the direct-to-LDS loads (per-token scales only).
    constexpr bool kSclLds = AB == 0;
    constexpr int kSclA = (BM * 4 + 1023) / 1024, kSclC = (BN * 4 + 1023) / 1024;
    __shared__ __attribute__((aligned(16))) uint8_t scl_a[kSclLds ? kSclA * 1024 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t scl_c[kSclLds ? kSclC * 1024 : 16];

    const int tid = threadIdx.x;
    // readfirstlane: the compiler then knows the wavefront index is uniform,
    // so LDS block addresses (m0 of the direct loads) stay in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int c = lane & 15;

    // Tile order: consecutive workgroup ids go round-robin over the 8 XCDs, so
    // each XCD gets a contiguous slice of a grouped traversal (4 row tiles per
    // group) and the workgroups sharing an L2 share activation rows and weights.
    const int64_t mtiles = (m + BM - 1) / BM;
    const int64_t ntb = (n + BN - 1) / BN;
    const int64_t nwg = mtiles * ntb;
    int64_t id = blockIdx.x;
    if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
    constexpr int64_t GM = 4;
    const int64_t group = id / (GM * ntb);
    const int64_t first_m = group * GM;
    const int64_t gsize = (mtiles - first_m < GM) ? (mtiles - first_m) : GM;
    const int64_t within = id - group * GM * ntb;
    const int64_t m0 = (first_m + within % gsize) * BM;
    const int64_t n0 = (within / gsize) * BN;
    const int64_t t0 = n0 / kNTile;
    const int64_t ntiles = n / kNTile;

    // This workgroup's K slice: the operand pointers move to its first chunk
    // (strides stay those of the whole K), its partials to slice blockIdx.y.
    const int64_t k0 = (int64_t)blockIdx.y * kslice;
    a_q += k0;
    w_packed += (k0 / kChunkK) * (WF == kW8 ? 2 * kChunkBytes : kChunkBytes);
    if (WF != kW8) grp_scale += (k0 / kGroup) * kNTile * (WF == kW4Lqq ? 2 : 1);
    out = (uint8_t *)out + (int64_t)blockIdx.y * m * ldo * (out_dtype == 1 ? 2 : 4);
    // K in whole 128-wide chunks plus at most one trailing 64-wide chunk (only
    // in the last slice).  All indices and offsets below fit 32 bits: k <=
    // K_MAX, and one workgroup reads at most BM k activation bytes and 16 BN k
    // weight bytes (< 2^26).
    const int kfull = (int)k;
    const int ki = (int)(k - k0 < kslice ? k - k0 : kslice);   // this slice
    const int nchunks = (ki + kChunkK - 1) / kChunkK;
    const int nfull = ki / kChunkK;
    const int gk = kfull / kGroup;
    const std::integral_constant<bool, true> full_chunk;
    const std::integral_constant<bool, false> half_chunk;
    const std::integral_constant<bool, true> steady;      // request offsets known whole
    const std::integral_constant<bool, false> general;

    // Buffer resources over this workgroup's rows of A and tiles of W: rows
    // past m and tiles past n read zero (they only reach unstored outputs), so
    // no per-lane clamp is needed; each chunk's offset goes in a scalar.
    constexpr int kWTileMul = WF == kW8 ? 16 : 8;                // weight bytes per tile = mul * k
    constexpr int kPSize = WF == kW4Lqq ? 2 : 1;                 // bytes per group parameter
    const int rows_here = (int)(m - m0 < BM ? m - m0 : BM);
    const int tiles_here = (int)(ntiles - t0 < NTB ? ntiles - t0 : NTB);
    const int wtile = kWTileMul * kfull;
    const int ptile = kNTile * gk * kPSize;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a_q + m0 * k, (uint32_t)rows_here * kfull);
    const __amdgpu_buffer_rsrc_t rw =
        buffer_rsrc(w_packed + t0 * (int64_t)wtile, (uint32_t)tiles_here * wtile);
    const __amdgpu_buffer_rsrc_t rp =
        WF == kW8 ? rw : buffer_rsrc(grp_scale + t0 * (int64_t)ptile, (uint32_t)tiles_here * ptile);

    // The epilogue's scales go to LDS before any chunk is requested, so they
    // are in long before the K loop ends; read from global memory at the
    // epilogue they would queue behind the output stores of every other
    // workgroup finishing the same round.  Rows past m and columns past n read
    // zero and are not stored.  These are the oldest loads of the wavefronts
    // that issue them, so every wait below covers them.
    if constexpr (kSclLds) {
        static_assert(WAVES >= kSclA + kSclC, "one scale block per wavefront");
        if (wave < kSclA) {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a_scale + m0, (uint32_t)rows_here * 4);
            buffer_to_lds16(rs, scl_a + wave * 1024, wave * 1024 + lane * 16, 0);
        } else if (wave < kSclA + kSclC) {
            const int b = wave - kSclA;
            const int cols_here = (int)(n - n0 < BN ? n - n0 : BN);
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(ch_scale + n0, (uint32_t)cols_here * 4);
            buffer_to_lds16(rs, scl_c + b * 1024, b * 1024 + lane * 16, 0);
        }
    }

    // Activations of chunk j -> stage buf, buffer -> LDS directly (one 1 KB
    // block = 8 rows of 128 bytes per instruction, 16-byte columns swizzled).
    // For the trailing 64-wide chunk the upper 64 columns are folded onto the
    // lower ones, so no load leaves the row; they are never read.
    int aoff[ACT_I];
#pragma unroll
    for (int i = 0; i < ACT_I; ++i) {
        const int row = (i * WAVES + wave) * 8 + (lane >> 3);
        aoff[i] = row * kfull + (act_swz(row, lane & 7) << 4);
    }
    // Stage and register-set selection by a compile-time tag (0, 1 or 2).
    auto act_of = [&](auto st) -> uint8_t * {
        constexpr int S = (int)decltype(st)::value;
        if constexpr (S == 0) return act0;
        else if constexpr (S == 1) return act1;
        else return act2;
    };
    auto issue_act = [&](int j, auto buf_tag, auto full_tag) {
        uint8_t *base = act_of(buf_tag);
#pragma unroll
        for (int i = 0; i < ACT_I; ++i) {
            const int blk = i * WAVES + wave;
            int off = aoff[i];
            if constexpr (!decltype(full_tag)::value)
                off -= (act_swz(blk * 8 + (lane >> 3), lane & 7) & 4) << 4;
            buffer_to_lds16(ra, base + blk * 1024, off, j * kChunkK);
        }
    };
    // Packed records and group-parameter words of this wavefront's tile(s) for
    // chunk j.  A trailing 64-wide chunk of a 4-bit format has 8-byte records:
    // the 16-byte window is kept inside the 512-byte chunk (lane 63 reads the
    // last 16 bytes) and the wanted half picked at the rebuild; its missing
    // second group reads the first group's word.  An int8 half chunk holds step
    // 0 only, reloaded in place of step 1.
    //
    // Two register sets, by parity of the chunk index: the records of chunk
    // j + 2 are requested at the start of iteration j, land during its MFMAs
    // and are rebuilt in iteration j + 1 (kRegW: three sets, see the K loop).
    // Requests past the last chunk are clamped to it (fetched, never used).
    int woff[TPW], woff_half[TPW], poff[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tr = wave * TPW + i;
        woff[i] = tr * wtile + lane * 16;
        woff_half[i] = tr * wtile + (lane * 8 < 496 ? lane * 8 : 496);
        poff[i] = tr * ptile + (WF == kW4Lqq ? (c & ~1) * 2 : (c & ~3));
    }
    const WParamSel psel = wparam_selectors<WF>(c);
    WRec<WF> wrec0[TPW], wrec1[TPW], wrec2[TPW];
    uint32_t wsc0[TPW][2], wsc1[TPW][2], wsc2[TPW][2];
    auto wrec_of = [&](auto st) -> WRec<WF>(&)[TPW] {
        constexpr int S = (int)decltype(st)::value;
        if constexpr (S == 0) return wrec0;
        else if constexpr (S == 1) return wrec1;
        else return wrec2;
    };
    auto wsc_of = [&](auto st) -> uint32_t(&)[TPW][2] {
        constexpr int S = (int)decltype(st)::value;
        if constexpr (S == 0) return wsc0;
        else if constexpr (S == 1) return wsc1;
        else return wsc2;
    };
    // With weights in registers (kRegW) each wavefront's tiles are read by this
    // workgroup only: their records are streamed with the nontemporal policy,
    // which keeps them from evicting the activation tiles that every column
    // tile re-reads from L2 (70B FFN-down M = 64, split K: 40.7 -> 35.8 us).
    // In the LDS-weight form a tile is shared by the workgroups of a column of
    // tiles, so its records are cached normally.
    auto wload = [&](int voff, int soff) -> u32x4 {
        if constexpr (kRegW) return buffer_load16_nt(rw, voff, soff);
        else return buffer_load16(rw, voff, soff);
    };
    // steady_tag true: jreq is known to be a full chunk (no clamp, no select).
    auto fetch_w = [&](int jreq, auto set_tag, auto steady_tag) {
        WRec<WF>(&wrec)[TPW] = wrec_of(set_tag);
        uint32_t(&wsc)[TPW][2] = wsc_of(set_tag);
        constexpr bool kSteady = decltype(steady_tag)::value;
        const int j = kSteady || jreq < nchunks ? jreq : nchunks - 1;
        const bool wfull = kSteady || j < nfull;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if constexpr (WF == kW8) {
                const int so = j * (2 * kChunkBytes);
                wrec[i].r0 = wload(woff[i], so);
                wrec[i].r1 = wload(woff[i], wfull ? so + kChunkBytes : so);
                wsc[i][0] = wsc[i][1] = 0u;
            } else {
                wrec[i].r = wload(wfull ? woff[i] : woff_half[i], j * kChunkBytes);
                const int so = j * (2 * kNTile * kPSize);
                wsc[i][0] = buffer_load4(rp, poff[i], so);
                wsc[i][1] = buffer_load4(rp, poff[i], wfull ? so + kNTile * kPSize : so);
            }
        }
    };
    // A trailing 64-wide chunk of a 4-bit format: pick this lane's 8-byte half
    // of the 16-byte window (see above) into the step-0 words.
    auto half_records = [&](auto set_tag) {
        if constexpr (WF != kW8) {
            WRec<WF>(&wrec)[TPW] = wrec_of(set_tag);
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                wrec[i].r = (lane == 63) ? u32x4{wrec[i].r.z, wrec[i].r.w, 0u, 0u}
                                         : u32x4{wrec[i].r.x, wrec[i].r.y, 0u, 0u};
        }
    };
    // Rebuild the int8 operands of both K steps of chunk j (from the register
    // set of its parity) into the LDS stage of the same parity.
    auto rebuild_w = [&](auto buf_tag, auto full_tag) {
        uint8_t *wbase = decltype(buf_tag)::value ? wl1 : wl0;
        WRec<WF>(&wrec)[TPW] = decltype(buf_tag)::value ? wrec1 : wrec0;
        uint32_t(&wsc)[TPW][2] = decltype(buf_tag)::value ? wsc1 : wsc0;
        if constexpr (!decltype(full_tag)::value) half_records(buf_tag);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tt = wave * TPW + i;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t mul = 0u, add = 0u;
                if constexpr (WF != kW8) wparam_consts<WF>(wsc[i][h], psel, mul, add);
                *(v4i *)(wbase + ((tt * 2 + h) * 64 + lane) * 16) =
                    wrec_operand_ma<WF>(wrec[i], h, mul, add);
            }
        }
    };

    v4i acc[TN][TM];
    f32x4 accf[AB ? TN : 1][AB ? TM : 1];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int jj = 0; jj < TM; ++jj) {
            acc[i][jj] = v4i{0, 0, 0, 0};
            if constexpr (AB > 0) accf[i][jj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }

    // Per-block activation scales of this lane's rows for one chunk (AB > 0),
    // fetched one chunk ahead like the operands.  Blocks past k (a trailing
    // half chunk) are clamped to the last block and never used.
    constexpr int NBC = AB ? kChunkK / AB : 1;
    float scur[AB ? TM : 1][NBC], snxt[AB ? TM : 1][NBC];
    const int64_t nblk = AB ? k / AB : 1;
    auto fetch_s = [&](int64_t j, float (&sdst)[AB ? TM : 1][NBC]) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int64_t row = m0 + wm * WM + tm * 16 + c;
            const int64_t rowc = row < m ? row : m - 1;
#pragma unroll
            for (int b = 0; b < NBC; ++b) {
                const int64_t blk = j * NBC + b < nblk ? j * NBC + b : nblk - 1;
                sdst[tm][b] = a_scale[rowc * nblk + blk];
            }
        }
    };

    // One K step (64) of stage buf: LDS reads and MFMAs only.  Activation
    // fragment: lane (c, kq) reads row c of the row tile at 16-byte column
    // 4 h + kq; weight fragments are stored in operand order.
    const int kq = lane >> 4;
    auto mma_step = [&](auto buf_tag, int h) {
        const uint8_t *abase = act_of(buf_tag);
        const uint8_t *wbase = decltype(buf_tag)::value ? wl1 : wl0;
        v4i av[TM], wv[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
            av[tm] = *(const v4i *)(abase + act_lds_off(wm * WM + tm * 16 + c, 4 * h + kq));
        if constexpr (kRegW) {
            const WRec<WF>(&wrec)[TPW] = wrec_of(buf_tag);
            const uint32_t(&wsc)[TPW][2] = wsc_of(buf_tag);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                uint32_t mul = 0u, add = 0u;
                if constexpr (WF != kW8) wparam_consts<WF>(wsc[tn][h], psel, mul, add);
                wv[tn] = wrec_operand_ma<WF>(wrec[tn], h, mul, add);
            }
        } else {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                wv[tn] = *(const v4i *)(wbase + (((wn * TN + tn) * 2 + h) * 64 + lane) * 16);
        }
        if constexpr (AB == 0) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    acc[tn][tm] = mfma16x16x64(wv[tn], av[tm], acc[tn][tm]);
        } else if constexpr (AB == 32) {
            const v4i zero = {0, 0, 0, 0};
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    fold4(accf[tn][tm], mfma16x16x64(wv[tn], half_operand(av[tm], kq, 0), zero),
                          scur[tm][2 * h]);
                    fold4(accf[tn][tm], mfma16x16x64(wv[tn], half_operand(av[tm], kq, 1), zero),
                          scur[tm][2 * h + 1]);
                }
        } else if constexpr (AB == 64) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    fold4(accf[tn][tm], mfma16x16x64(wv[tn], av[tm], v4i{0, 0, 0, 0}),
                          scur[tm][h]);
        } else {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    // the block's first K step starts from a zero accumulator
                    // (inline constant), so no register clearing after the fold
                    // (prefill, block 128: 407 -> 381 us)
                    acc[tn][tm] =
                        mfma16x16x64(wv[tn], av[tm], h == 0 ? v4i{0, 0, 0, 0} : acc[tn][tm]);
                    if (h == 1) fold4(accf[tn][tm], acc[tn][tm], scur[tm][0]);
                }
        }
    };

    // Workgroup barrier for the LDS stages: wait until this wavefront's LDS
    // writes and vector-memory loads (including the direct-to-LDS ones) are
    // done, then s_barrier.  The empty asm statements keep the compiler from
    // moving memory accesses across it.
#define W4A8_LDS_BARRIER()                                                               \
    do {                                                                                \
        __builtin_amdgcn_s_waitcnt(0);                                                  \
        asm volatile("" ::: "memory");                                                  \
        __builtin_amdgcn_s_barrier();                                                   \
        asm volatile("" ::: "memory");                                                  \
    } while (0)

    // Pipeline over K chunks: iteration j multiplies stage `cur` while stage
    // `nxt` is filled for chunk j + 1.  It runs the first K step of chunk j,
    // then sends its memory requests (the direct-to-LDS activation loads of
    // chunk j + 1 and the weight records of chunk j + 2), runs the second K
    // step, rebuilds this wavefront's weight tile(s) of chunk j + 1 into `nxt`
    // from records requested one iteration earlier, and ends on a barrier that
    // waits for every request of the iteration.  So a rebuild only reads
    // registers that a barrier's wait already covered: with direct-to-LDS
    // loads in flight the compiler cannot count vector loads in order, and any
    // earlier use of a loaded register would make it wait for all of them, the
    // activation loads just issued included.
    //   The order is measured (70B FFN-down, 2048 x 8192 x 28672, interleaved
    // runs on three boxes: 386-397 -> 367-381 us).  The first K step's LDS
    // reads go out alone right after the barrier, ahead of the activation
    // loads that also write LDS; the two K steps run back to back; the
    // wavefront runs its MFMA steps at a raised priority (s_setprio) and drops
    // it for the rebuild, so on each SIMD the wavefronts still multiplying
    // win the issue arbitration over those that have reached their VALU work.
    // The scheduling barriers keep the compiler from moving work across these
    // phases.
    const std::integral_constant<bool, false> stage0;
    const std::integral_constant<bool, true> stage1;
    // kRegW: vector-memory requests one chunk makes (activation blocks, then
    // per tile a record and two parameter words, or two int8 records).  The
    // barrier waits until at most that many remain: loads complete in order,
    // so that is exactly the older chunk, and the newer one stays in flight.
    constexpr int kChunkReq = ACT_I + TPW * (WF == kW8 ? 2 : 3);
    static_assert(!kRegW || (AB == 0 && kChunkReq < 64), "one chunk of requests in flight");
    constexpr int kWaitOlder = (kChunkReq & 15) | ((kChunkReq >> 4) << 14) | 0x70;  // lgkmcnt 0
    const std::integral_constant<int, 2> stage2;
    if constexpr (kRegW) {
        if (nchunks > 0) {
            if (nfull > 0) issue_act(0, stage0, full_chunk);
            else issue_act(0, stage0, half_chunk);
            fetch_w(0, stage0, general);
            // every request of chunk 0 before any of chunk 1: the wait below
            // counts on that order
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            // chunk 1, or chunk 0 again when there is no chunk 1 (never used)
            const int j1 = nchunks > 1 ? 1 : 0;
            if (j1 < nfull) issue_act(j1, stage1, full_chunk);
            else issue_act(j1, stage1, half_chunk);
            fetch_w(1, stage1, general);
        }
        __builtin_amdgcn_s_waitcnt(kWaitOlder);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    } else {
        if (nchunks > 0) {
            fetch_w(0, stage0, general);
            fetch_w(1, stage1, general);
            if (nfull > 0) {
                rebuild_w(stage0, full_chunk);
                issue_act(0, stage0, full_chunk);
            } else {
                rebuild_w(stage0, half_chunk);
                issue_act(0, stage0, half_chunk);
            }
            if constexpr (AB > 0) fetch_s(0, scur);
        }
        W4A8_LDS_BARRIER();
    }
    auto iteration = [&](int j, auto cur, auto nxt) {
        __builtin_amdgcn_s_setprio(2);
        mma_step(cur, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < nfull) issue_act(j + 1, nxt, full_chunk);
        else if (j + 1 < nchunks) issue_act(j + 1, nxt, half_chunk);
        fetch_w(j + 2, cur, general);
        if constexpr (AB > 0)
            if (j + 1 < nchunks) fetch_s(j + 1, snxt);
        __builtin_amdgcn_sched_barrier(0);
        if (j < nfull) mma_step(cur, 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (j + 1 < nfull) rebuild_w(nxt, full_chunk);
        else if (j + 1 < nchunks) rebuild_w(nxt, half_chunk);
        W4A8_LDS_BARRIER();
        if constexpr (AB > 0) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int b = 0; b < NBC; ++b) scur[tm][b] = snxt[tm][b];
        }
    };
    // kRegW: three stages, two chunks ahead.  Iteration j requests the
    // activations and weight records of chunk j + 2 into the stage and
    // register set that chunk j - 1 used, multiplies chunk j with its
    // operands rebuilt in registers from the records of its set, and ends on
    // a barrier that waits for chunk j + 1's requests only.  Requests past
    // the last chunk are clamped to it (every address stays inside the
    // operands) and land in a stage and set that are not used again.
    //   In the steady state (steady_tag true: chunks j .. j + 2 all whole) the
    // requests take fixed offsets.  Otherwise the clamp and the whole / half
    // choice are selects, whose results the register allocator may place in
    // a register set that a load still in flight will write; the compiler
    // then waits for that load before the select, which had cut the requests
    // in flight to one chunk in every third iteration.
    //   Two workgroups share each CU in the split-K launch, and the issue
    // arbiter favours the older wavefronts: the first-started workgroup of a
    // pair ran its K loop in 17.4-18.0 us, the second in 21.8-22.3 us (70B
    // FFN-down M = 64, per-workgroup stamps).  The pair takes turns at a
    // raised wave priority, chunk by chunk, so both progress together (two
    // boxes, interleaved: fused M = 64 39.9-40.4 -> 39.3-39.4 us, split GEMM
    // M = 64 36.3 -> 35.5 us, M = 32 30.8-31.2 -> 29.9-30.5 us).
    const bool second =
        (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x >= first_wave;
    auto iteration_rw = [&](int j, auto cur, auto ahead, auto steady_tag) {
        if ((j + (int)second) & 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        if constexpr (decltype(steady_tag)::value) {
            issue_act(j + 2, ahead, full_chunk);
            fetch_w(j + 2, ahead, steady_tag);
        } else {
            const int ja = j + 2 < nchunks ? j + 2 : nchunks - 1;
            if (ja < nfull) issue_act(ja, ahead, full_chunk);
            else issue_act(ja, ahead, half_chunk);
            fetch_w(j + 2, ahead, steady_tag);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!decltype(steady_tag)::value && j >= nfull) half_records(cur);
        mma_step(cur, 0);
        if (decltype(steady_tag)::value || j < nfull) mma_step(cur, 1);
        __builtin_amdgcn_s_waitcnt(kWaitOlder);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    if constexpr (kRegW) {
        int j = 0;
        for (; j + 4 < nfull; j += 3) {
            iteration_rw(j, stage0, stage2, steady);
            iteration_rw(j + 1, stage1, stage0, steady);
            iteration_rw(j + 2, stage2, stage1, steady);
        }
        for (; j < nchunks; j += 3) {
            iteration_rw(j, stage0, stage2, general);
            if (j + 1 < nchunks) iteration_rw(j + 1, stage1, stage0, general);
            if (j + 2 < nchunks) iteration_rw(j + 2, stage2, stage1, general);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        for (int j = 0; j < nchunks; j += 2) {
            iteration(j, stage0, stage1);
            if (j + 1 < nchunks) iteration(j + 1, stage1, stage0);
        }
    }
    // the clamped requests past the last chunk: done before the stages are reused
    W4A8_LDS_BARRIER();
#undef W4A8_LDS_BARRIER

    // Epilogue through LDS (free after the last barrier): each wavefront writes
    // its WM x WN tile of final values (bf16, fp32 or int32) to its own slice of
    // the stage arrays, then stores whole 128-byte row segments, so each output
    // cache line is written in full (straight from the accumulator layout a lane
    // holds only 4 consecutive columns of a row).  16-byte segments are
    // XOR-swizzled by the row (mod 8, or mod the segments per row when a row
    // has fewer) for conflict-free reads.  Four-byte outputs go in
    // two passes of half the rows.
    {
        constexpr int PER_ARRAY = WAVES / 4;
        static_assert(WAVES % 4 == 0, "four stage arrays share the epilogue");
        const int esize = (out_dtype == 1) ? 2 : 4;
        const int rows_pass = (esize == 2) ? WM : WM / 2;
        const int row_bytes = WN * esize;
        const int segs = row_bytes / 16;                 // 16-byte segments per row
        // kRegW: the weight stages held no operands; half the wavefronts use each
        constexpr int PER_W = WAVES / 2;
        static_assert(kRegW ? WM * WN * 2 * PER_W <= kEpiW
                            : WM * WN * 2 <= (L::kW < L::kAct ? L::kW : L::kAct) / PER_ARRAY,
                      "epilogue tile fits the stage arrays");
        const int which = wave / PER_ARRAY;
        uint8_t *ebuf =
            kRegW ? (wave < PER_W ? wl0 : wl1) + (wave % PER_W) * (WM * WN * 2)
                  : (which == 0 ? act0 : which == 1 ? act1 : which == 2 ? wl0 : wl1) +
                        (wave % PER_ARRAY) * (WM * WN * 2);
        // the XOR stays inside the row: segs is a power of two, 2 to 16
        const int swz_mask = (segs < 8 ? segs : 8) - 1;
        auto seg_off = [&](int r, int seg) {
            return r * row_bytes + ((seg ^ (r & swz_mask)) << 4);
        };
        // channel scales of this lane's 4 columns per 16-column tile (past n:
        // zero or clamped; those columns are not stored)
        f32x4 scv[TN];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int col = wn * WN + tn * 16 + 4 * kq;
            if constexpr (kSclLds) {
                scv[tn] = *(const f32x4 *)(scl_c + col * 4);
            } else {
                const int64_t nn = n0 + col;
                scv[tn] = *(const f32x4 *)(ch_scale + (nn < n ? nn : n - 4));
            }
        }
        for (int pass = 0; pass < WM / rows_pass; ++pass) {
            // accumulators -> LDS (lane (c, kq): row tm * 16 + c, 4 columns)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int r = tm * 16 + c - pass * rows_pass;
                if (r < 0 || r >= rows_pass) continue;
                const float sa =
                    AB ? 1.0f : *(const float *)(scl_a + (wm * WM + tm * 16 + c) * 4);
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const int col = tn * 16 + 4 * kq;             // within the wavefront tile
                    const int byte = col * esize;
                    uint8_t *dst = ebuf + seg_off(r, byte >> 4) + (byte & 15);
                    const v4i a4 = acc[tn][tm];
                    if (!AB && out_dtype == 2) {
                        *(v4i *)dst = a4;
                    } else {
                        const f32x4 sc = scv[tn];
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (AB > 0) {
                                y[i] = accf[tn][tm][i] * sc[i];
                            } else {
                                y[i] = (float)a4[i] * sa;
                                y[i] = y[i] * sc[i];
                            }
                        }
                        if (out_dtype == 1)
                            *(u32x2 *)dst = u32x2{bf16x2_rne(y[0], y[1]),
                                                  bf16x2_rne(y[2], y[3])};
                        else
                            *(f32x4 *)dst = f32x4{y[0], y[1], y[2], y[3]};
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wavefront's LDS writes done
            asm volatile("" ::: "memory");
            // LDS -> global: 16 bytes per lane, whole rows of the wavefront tile
            const int lanes_per_row = segs;               // 8 (bf16) or 16 (4-byte)
            const int rows_per_iter = 64 / lanes_per_row;
            for (int r0 = 0; r0 < rows_pass; r0 += rows_per_iter) {
                const int r = r0 + lane / lanes_per_row;
                const int seg = lane % lanes_per_row;
                const int64_t row = m0 + wm * WM + pass * rows_pass + r;
                const int64_t nn = n0 + wn * WN + (seg * 16) / esize;
                const u32x4 v = *(const u32x4 *)(ebuf + seg_off(r, seg));
                if (row < m && nn < n)
                    *(u32x4 *)((uint8_t *)out + (row * ldo + nn) * esize) = v;
            }
            asm volatile("" ::: "memory");
        }
    }
}

template <int WF, int MT, int NT, bool FUSED, int AV = 1, int AB = 0, int FW = 8, bool KF = false>
void launch_skinny(const void *act, const float *a_scale, const uint8_t *w_packed,
                   const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                   int64_t k, void *out, int out_dtype, int8_t *ws_q, float *ws_s,
                   size_t dyn_lds, hipStream_t stream) {
    // chunks per load batch: fewer when each batch also carries MT activation
    // tiles.  The fused form runs FW wavefronts (fused_waves: 16 give its
    // quantization prologue, which every workgroup runs over all of A, four
    // wavefronts per SIMD; 8 take deeper batches of the weight stream), and
    // with two tiles per workgroup batches of two chunks.
    constexpr int WAVES = FUSED ? FW : 8,
                  D = FUSED ? (FW == 16 || NT == 2 ? 2 : 4)
                            : (MT == 1 ? 4 : (MT == 2 ? 2 : (NT == 1 && AB == 0 ? 2 : 1)));
    const int64_t ntiles = n / kNTile;
    const unsigned grid = (unsigned)((ntiles + NT - 1) / NT);
    gemm_skinny_kernel<WF, MT, NT, WAVES, D, FUSED, AV, AB, KF><<<grid, 64 * WAVES, dyn_lds,
                                                            stream>>>(
        act, a_scale, w_packed, grp_scale, ch_scale, (int)m, n, k, out, out_dtype, ws_q, ws_s,
        (int64_t)device_cu_count());
}

// Output columns [n_off, n_off + n_sub) of an [m, ldo] product: the weight
// pointers move by whole 16-channel tiles (tile-major layouts).  kslice > 0
// splits K into ceil(k / kslice) slices of int32 partials (see the kernel).
template <int WF, int BM, int BN, int WAVES_M, int WAVES_N, int AB = 0>
void launch_tiled_cols(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                       const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n_off,
                       int64_t n_sub, int64_t ldo, int64_t k, void *out, int out_dtype,
                       hipStream_t stream, int64_t kslice = 0) {
    if (n_sub <= 0) return;
    if (kslice <= 0 || kslice >= k) kslice = k;
    const int64_t t_off = n_off / kNTile;
    const int64_t wtile = WF == kW8 ? kNTile * k : kNTile * k / 2;      // bytes per tile
    const int64_t ptile = kNTile * (k / kGroup) * (WF == kW4Lqq ? 2 : 1);  // parameter bytes
    const int esize = out_dtype == 1 ? 2 : 4;
    const int64_t grid = ((m + BM - 1) / BM) * ((n_sub + BN - 1) / BN);
    // k == 0: one slice of no chunks (the product is zero)
    const unsigned slices = kslice > 0 ? (unsigned)((k + kslice - 1) / kslice) : 1u;
    gemm_tiled_kernel<WF, BM, BN, WAVES_M, WAVES_N, AB><<<dim3((unsigned)grid, slices),
                                                          64 * WAVES_M * WAVES_N, 0, stream>>>(
        a_q, a_scale, w_packed + t_off * wtile,
        grp_scale ? grp_scale + t_off * ptile : grp_scale, ch_scale + n_off, m, n_sub, k,
        (uint8_t *)out + n_off * esize, ldo, out_dtype, kslice, (int64_t)device_cu_count());
}

// ------------------------------------------------------------- split K --
// The skinny kernel's wavefronts split K inside one workgroup per 16-channel
// tile, so every workgroup reads all of A: at m = 64, k = 28672 that is 470 MB
// of activation loads for 117 MB of weights, and the vector-memory address
// path of the CUs, not HBM, sets the time.  With a caller workspace, such
// shapes instead run 64 x 128 output tiles of the tiled kernel (A shared by its
// 8 wavefronts through LDS; rows past m read zero) over S slices of K, each
// slice writing int32 partials, then a pass that sums the slices (exact, any
// order) and applies the same binary32 epilogue as the one-pass kernels.
constexpr int kSplitBM = 64, kSplitBN = 128;
// Batches of 65 rows and more whose 128 x 256 tiles number fewer than the
// CUs: the one-pass kernels leave CUs idle (8192 x 28672, same box: m = 128 222
// us, m = 256 182 us, against 36 us at m = 64 split), so K is split over
// 128 x 256 tiles (the weights-in-registers form, one workgroup per CU).
constexpr int kSplitMidBM = 128, kSplitMidBN = 256;
constexpr int64_t kSplitMidWgs = 256;
// Partials this small stay in the caches: more slices than twice the weight
// bytes allow, for long enough K (A/B on MI355X, HIP events: 1024 x 8192 at
// m = 768 58.0 -> 26.0 us, 5120 x 5120 at m = 384 41.8 -> 29.3, 4096 x 4096 at
// m = 512 34.1 -> 27.2; at k = 2048 with 64 tiles or more the finalize pass
// costs more than it saves: 8192 x 2048 at m = 384 22.2 -> 25.0).
constexpr int64_t kSplitMidL2 = (int64_t)64 << 20;

// Up to 64 rows, whether K is split at all comes from a model of the two
// paths' times (ns, integers scaled to stay exact), fitted to MI355X
// measurements of both over 46 shapes (m 5..64, n and k 1024..28672):
//   one pass: 1500 + R k (300 + 28 m) / 1000, R = ceil(W / 256) rounds of its
//             W workgroups (one 16-channel tile each; two for m > 32 and at
//             least 512 tiles), each reading all of A through the vector
//             memory path, which sets its pace;
//   split:    7400 + 360 C max(256, G) / 256, C chunks per slice, G = S
//             ceil(n / 128) workgroups (a fixed cost for the two launches,
//             the sliced kernel and the sum pass, and the pipeline fill;
//             then a chunk per 360 ns per CU);
// K is split when the split model is below 0.9 of the one-pass model.  Over
// the measured shapes the choice costs 0.5 % against the faster path of each
// (the rule before it: 20 %); its worst pick is 13 % slower (48 x 13824 x 3072).
inline bool splitk_small_pays(int64_t m, int64_t n, int64_t k, int64_t s) {
    const int64_t ntb = (n + kSplitBN - 1) / kSplitBN;
    const int64_t chunks = (k / kChunkK + s - 1) / s;
    const int64_t wgs = ntb * s;
    const __int128 t_split = (__int128)7400 * 256 + (__int128)360 * chunks * (wgs > 256 ? wgs : 256);
    const int64_t ntiles = n / kNTile;
    const int64_t per_wg = (m > 32 && ntiles >= 512) ? 2 : 1;
    const int64_t rounds = ((ntiles + per_wg - 1) / per_wg + kSplitMidWgs - 1) / kSplitMidWgs;
    const __int128 t_one = (__int128)1500 * 1000 + (__int128)rounds * k * (300 + 28 * m);
    // t_split / 256 < 0.9 t_one / 1000
    return t_split * 10000 < t_one * 2304;
}

// Slices of K for an m x n x k split-K product (0: not split).  Up to 64 rows
// (from 5; the rows of a 64-row tile past m cost MFMA work but no memory
// traffic): 64 x 128 tiles, about 512 workgroups (two per CU: one alone leaves
// too few loads in flight), at most 16 slices of at least one chunk.  The
// partials cost 8 S m n bytes (written, then read) against n k / 2 bytes of
// 4-bit weights: S is cut to keep them within half the weights (32 S m <= k).
// For 16 < m with no cut, K is split; otherwise only where splitk_small_pays.
// More rows: the 128 x 256 form.
inline int64_t splitk_slices(int64_t m, int64_t n, int64_t k) {
    if (m < 5 || k < 2 * kChunkK) return 0;
    const int64_t nfull = k / kChunkK;
    if (m > 64) {
        // 128 x 256 tiles with weights in registers (one workgroup per CU):
        // split while the tiles alone would leave CUs idle, into at most one
        // round of kSplitMidWgs workgroups, with the partials within twice
        // the weight bytes (8 S m n <= n k) or kSplitMidL2 (k >= 4096, or
        // k >= 2048 with at most 32 tiles), slices of at least 4 chunks
        const int64_t tiles = ((m + kSplitMidBM - 1) / kSplitMidBM) *
                              ((n + kSplitMidBN - 1) / kSplitMidBN);
        int64_t s = kSplitMidWgs / tiles;
        int64_t cap = k / (8 * m);
        if ((nfull >= 32 || (nfull >= 16 && tiles <= 32)) && cap < kSplitMidL2 / (8 * m * n))
            cap = kSplitMidL2 / (8 * m * n);
        if (s > cap) s = cap;
        if (s > nfull / 4) s = nfull / 4;
        if (s > 16) s = 16;
        return s >= 2 ? s : 0;
    }
    const int64_t ntb = (n + kSplitBN - 1) / kSplitBN;
    int64_t s = (512 + ntb - 1) / ntb;
    if (s > nfull) s = nfull;
    if (s > 16) s = 16;
    if (m > 16 && 32 * s * m <= k) return s >= 2 ? s : 0;
    if (s > k / (32 * m)) s = k / (32 * m);
    if (s < 2) return 0;
    return splitk_small_pays(m, n, k, s) ? s : 0;
}
inline int64_t splitk_kslice(int64_t k, int64_t s) {
    const int64_t nfull = k / kChunkK;
    return ((nfull + s - 1) / s) * kChunkK;             // whole chunks per slice
}
// Bytes of int32 partials (0 when the shape is not split).
inline size_t splitk_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const int64_t s = splitk_slices(m, n, k);
    if (s == 0) return 0;
    const int64_t used = (k + splitk_kslice(k, s) - 1) / splitk_kslice(k, s);
    return (size_t)used * (size_t)m * (size_t)n * 4;
}

// out[r][c..c+3] from the sum of the int32 partial slices [slices][m][n].  With
// S > 0 the count is a template argument (S == slices), so a thread's S loads
// are all in flight before the first add; a runtime trip count (S == 0) left
// them one round trip apart.
template <int S>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const v4i *__restrict__ part,
                                                              int slices, int64_t m, int64_t n,
                                                              const float *__restrict__ a_scale,
                                                              const float *__restrict__ ch_scale,
                                                              void *__restrict__ out, int out_dtype) {
    const int64_t quads = m * (n / 4);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
        v4i acc;
        if constexpr (S > 0) {
            v4i p[S];
#pragma unroll
            for (int s = 0; s < S; ++s) p[s] = part[s * quads + q];
            acc = p[0];
#pragma unroll
            for (int s = 1; s < S; ++s)
                acc = v4i{acc[0] + p[s][0], acc[1] + p[s][1], acc[2] + p[s][2], acc[3] + p[s][3]};
        } else {
            acc = part[q];
            for (int s = 1; s < slices; ++s) {
                const v4i p = part[s * quads + q];
                acc = v4i{acc[0] + p[0], acc[1] + p[1], acc[2] + p[2], acc[3] + p[3]};
            }
        }
        const int64_t row = q / (n / 4), col = (q - row * (n / 4)) * 4;
        store4(out, out_dtype, row, n, col, acc, a_scale[row], *(const f32x4 *)(ch_scale + col));
    }
}

// Unrolled forms for 2..17 slices (splitk_slices gives at most 16, plus one
// slice for a trailing half chunk); any other count takes the runtime loop.
template <int S>
void launch_finalize(const int32_t *partials, int slices, int64_t m, int64_t n,
                     const float *a_scale, const float *ch_scale, void *out, int out_dtype,
                     unsigned grid, hipStream_t stream) {
    if constexpr (S > 17) {
        splitk_finalize_kernel<0><<<grid, 256, 0, stream>>>((const v4i *)partials, slices, m, n,
                                                            a_scale, ch_scale, out, out_dtype);
    } else {
        if (slices == S)
            splitk_finalize_kernel<S><<<grid, 256, 0, stream>>>((const v4i *)partials, slices, m,
                                                                n, a_scale, ch_scale, out,
                                                                out_dtype);
        else
            launch_finalize<S + 1>(partials, slices, m, n, a_scale, ch_scale, out, out_dtype, grid,
                                   stream);
    }
}

template <int WF>
void launch_splitk(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                   const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                   int64_t k, void *out, int out_dtype, int32_t *partials, hipStream_t stream) {
    const int64_t s = splitk_slices(m, n, k);
    const int64_t kslice = splitk_kslice(k, s);
    const int slices = (int)((k + kslice - 1) / kslice);
    if (m > kSplitBM)
        launch_tiled_cols<WF, kSplitMidBM, kSplitMidBN, 1, 8>(a_q, a_scale, w_packed, grp_scale,
                                                              ch_scale, m, 0, n, n, k, partials, 2,
                                                              stream, kslice);
    else
        launch_tiled_cols<WF, kSplitBM, kSplitBN, 1, 8>(a_q, a_scale, w_packed, grp_scale,
                                                        ch_scale, m, 0, n, n, k, partials, 2,
                                                        stream, kslice);
    const int64_t quads = m * (n / 4);
    int64_t grid = (quads + 255) / 256;
    if (grid > 4096) grid = 4096;
    launch_finalize<2>(partials, slices, m, n, a_scale, ch_scale, out, out_dtype, (unsigned)grid,
                       stream);
}

template <int WF, int BM, int BN, int WAVES_M, int WAVES_N, int AB = 0>
void launch_tiled(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                  const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                  int64_t k, void *out, int out_dtype, hipStream_t stream) {
    launch_tiled_cols<WF, BM, BN, WAVES_M, WAVES_N, AB>(a_q, a_scale, w_packed, grp_scale,
                                                        ch_scale, m, 0, n, n, k, out, out_dtype,
                                                        stream);
}

// Large products: whole rounds of 256 x 256 tiles (one workgroup per compute
// unit) over a leading range of output columns, and the remaining columns in
// 128 x 256 tiles, half the work each, when that shortens the last round
// (e.g. 896 tiles on 256 compute units: 3 rounds of large tiles + half a round
// of small ones instead of 4 rounds).
template <int WF>
void launch_tiled_large(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                        const uint8_t *grp_scale, const float *ch_scale, int64_t m, int64_t n,
                        int64_t k, void *out, int out_dtype, hipStream_t stream) {
    const int ncu = device_cu_count();
    const int64_t mt = (m + 255) / 256, ntb = (n + 255) / 256;
    auto rounds = [&](int64_t tiles) { return (tiles + ncu - 1) / ncu; };
    // cost in units of one round of large tiles; large-tile columns first
    int64_t best_cols = ntb;
    double best = (double)rounds(mt * ntb);
    for (int64_t cols = ntb - 1; cols >= 0; --cols) {
        const double c = (double)rounds(mt * cols) + 0.5 * (double)rounds(2 * mt * (ntb - cols));
        if (c < best - 1e-9) {
            best = c;
            best_cols = cols;
        }
    }
    const int64_t n_large = best_cols * 256 < n ? best_cols * 256 : n;
    launch_tiled_cols<WF, 256, 256, 4, 4>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, 0,
                                          n_large, n, k, out, out_dtype, stream);
    // the tail as one row of 8 wavefronts of 128 x 32: weights unpacked in
    // registers (half the LDS writes of a 2 x 4 layout with LDS weights)
    launch_tiled_cols<WF, 128, 256, 1, 8>(a_q, a_scale, w_packed, grp_scale, ch_scale, m,
                                          n_large, n - n_large, n, k, out, out_dtype, stream);
}

// Largest m * (k + 16) the fused skinny prologue keeps in LDS, and the vectors
// per thread it holds in registers.
constexpr int64_t kFusedLdsMax = 48 * 1024;

// Activation vectors per thread the fused prologue needs for m rows of k
// (0 if the fused form does not apply).
[[maybe_unused]] int fused_vectors(int64_t m, int64_t n, int64_t k, int64_t ncu) {
    if (m < 1 || m > 16 || k < kChunkK) return 0;
    if (m * (k + 16) > kFusedLdsMax) return 0;
    const int64_t need = fused_need(m, k, fused_waves(m, n, k, ncu));
    return need <= 4 ? 4 : need <= kSkinnyMaxVec ? 8 : 0;
}

// GEMM on int8 activations for weight format WF.
template <int WF>
hipError_t launch_gemm_fmt(const int8_t *a_q, const float *a_scale, const uint8_t *w_packed,
                            const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                            int64_t n, int64_t k, void *out, int out_dtype,
                            hipStream_t stream, int32_t *partials = nullptr) {
    if (m == 0 || n == 0) return hipSuccess;
    const int64_t ntiles = n / kNTile;
    if (partials && splitk_slices(m, n, k) > 0) {
        // caller workspace of splitk_workspace_bytes(m, n, k) for the partials
        launch_splitk<WF>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k, out, out_dtype,
                          partials, stream);
    } else if (k < kChunkK) {
        // no full 128-wide chunk: the skinny kernel's loads assume one
        launch_tiled<WF, 128, 128, 2, 2>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k,
                                         out, out_dtype, stream);
    } else if (m <= 16) {
        launch_skinny<WF, 1, 1, false>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k, out,
                                   out_dtype, nullptr, nullptr, 0, stream);
    } else if (m <= 32) {
        launch_skinny<WF, 2, 1, false>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k, out,
                                   out_dtype, nullptr, nullptr, 0, stream);
    } else if (m <= 64) {
        if (ntiles >= 512)
            launch_skinny<WF, 4, 2, false>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k,
                                       out, out_dtype, nullptr, nullptr, 0, stream);
        else
            launch_skinny<WF, 4, 1, false>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k,
                                       out, out_dtype, nullptr, nullptr, 0, stream);
    } else if (m <= 128) {
        launch_tiled<WF, 128, 128, 2, 2>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k, out,
                               out_dtype, stream);
    } else {
        launch_tiled_large<WF>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n, k, out,
                               out_dtype, stream);
    }
    return hipGetLastError();
}

// Per-token quantization of bf16 activations into (ws_q, ws_s) and the GEMM;
// small m runs both in one kernel.
template <int WF>
hipError_t launch_gemm_bf16act_fmt(const uint16_t *a, const uint8_t *w_packed,
                                    const uint8_t *grp_scale, const float *ch_scale, int64_t m,
                                    int64_t n, int64_t k, void *out, int out_dtype,
                                    int8_t *ws_q, float *ws_s, hipStream_t stream,
                                    int32_t *partials = nullptr) {
    if (m == 0 || n == 0) return hipSuccess;
    const int ncu = device_cu_count();
    const int av = fused_vectors(m, n, k, ncu);
    if (av > 0) {
        const size_t lds_bytes = (size_t)(m * (k + 16));
        const bool w16 = fused_waves(m, n, k, ncu) == 16;
        // one workgroup per 16-channel tile: at most one per CU -> keep the floats
        const bool one_per_cu = n / kNTile <= (int64_t)ncu;
        if (av == 4 && w16 && one_per_cu)
            launch_skinny<WF, 1, 1, true, 4, 0, 16, true>(a, nullptr, w_packed, grp_scale, ch_scale,
                                                          m, n, k, out, out_dtype, ws_q, ws_s,
                                                          lds_bytes, stream);
        else if (av == 4 && w16)
            launch_skinny<WF, 1, 1, true, 4, 0, 16>(a, nullptr, w_packed, grp_scale, ch_scale, m,
                                                    n, k, out, out_dtype, ws_q, ws_s, lds_bytes,
                                                    stream);
        else if (w16)
            launch_skinny<WF, 1, 1, true, 8, 0, 16>(a, nullptr, w_packed, grp_scale, ch_scale, m,
                                                    n, k, out, out_dtype, ws_q, ws_s, lds_bytes,
                                                    stream);
        else if (av == 4 && fused_two_tiles(m, n, k, ncu))
            launch_skinny<WF, 1, 2, true, 4, 0, 8>(a, nullptr, w_packed, grp_scale, ch_scale, m, n,
                                                   k, out, out_dtype, ws_q, ws_s, lds_bytes, stream);
        else if (av == 4)
            launch_skinny<WF, 1, 1, true, 4, 0, 8>(a, nullptr, w_packed, grp_scale, ch_scale, m, n,
                                                   k, out, out_dtype, ws_q, ws_s, lds_bytes, stream);
        else
            launch_skinny<WF, 1, 1, true, 8, 0, 8>(a, nullptr, w_packed, grp_scale, ch_scale, m, n,
                                                   k, out, out_dtype, ws_q, ws_s, lds_bytes, stream);
        return hipGetLastError();
    }
    hipError_t e = launch_quantize_act(a, m, k, (int32_t)k, ws_q, ws_s, stream);
    if (e != hipSuccess) return e;
    return launch_gemm_fmt<WF>(ws_q, ws_s, w_packed, grp_scale, ch_scale, m, n, k, out,
                               out_dtype, stream, partials);
}

// GEMM with per-block activation scales (AB = 32, 64 or 128) on int8
// activations; output binary32 or bf16.
template <int WF, int AB>
hipError_t launch_gemm_blockact_fmt(const int8_t *a_q, const float *a_scale,
                                    const uint8_t *w_packed, const uint8_t *grp_scale,
                                    const float *ch_scale, int64_t m, int64_t n, int64_t k,
                                    void *out, int out_dtype, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (k < kChunkK)
        launch_tiled<WF, 128, 128, 2, 2, AB>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n,
                                             k, out, out_dtype, stream);
    else if (m <= 16)
        launch_skinny<WF, 1, 1, false, 1, AB>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n,
                                              k, out, out_dtype, nullptr, nullptr, 0, stream);
    else if (m <= 32)
        launch_skinny<WF, 2, 1, false, 1, AB>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n,
                                              k, out, out_dtype, nullptr, nullptr, 0, stream);
    else if (m <= 64)
        launch_skinny<WF, 4, 1, false, 1, AB>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n,
                                              k, out, out_dtype, nullptr, nullptr, 0, stream);
    else
        launch_tiled<WF, 128, 128, 2, 2, AB>(a_q, a_scale, w_packed, grp_scale, ch_scale, m, n,
                                             k, out, out_dtype, stream);
    return hipGetLastError();
}

}  // namespace
}  // namespace w4a8
