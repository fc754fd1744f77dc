// device_common.hpp -- helpers shared by the gfx950 kernels of libw4a8.so.
//
// Packed weight layout V1 (written by pack_w4_grouped, read by the GEMMs):
//   Output channels are grouped in tiles of 16 (t = n / 16, c = n % 16) and K
//   in chunks of 128 (j = k / 128; the last chunk is 64 wide when k % 128 == 64).
//   Inside a chunk, the 64 lanes of a wavefront each own one record:
//     lane = c + 16 * kq,   kq = (k % 64) / 16
//   A full chunk stores 16 bytes per lane (record at lane * 16): bytes 0..7 hold
//   the 16 weights of K-step h = 0 (k % 128 < 64), bytes 8..15 those of h = 1.
//   A half chunk stores 8 bytes per lane (record at lane * 8), step 0 only.
//   The 8 bytes of one step are two 32-bit words P0, P1; with e = k % 16:
//     e = 0..3   -> low  nibble of byte e     of P0
//     e = 4..7   -> high nibble of byte e - 4 of P0
//     e = 8..11  -> low  nibble of byte e - 8 of P1
//     e = 12..15 -> high nibble of byte e - 12 of P1
//   so (P & 0x0F0F0F0F) and ((P >> 4) & 0x0F0F0F0F) are four consecutive k in
//   byte order: exactly the 16-byte per-lane operand of v_mfma_i32_16x16x64_i8
//   for 16 output channels and 64 k.  A tile occupies 16 * k / 2 bytes and
//   chunk j starts at byte j * 1024 of its tile.
//   Nibbles hold u = q + 8 (q in [-7, 7]).
// Group scales in kernel order: byte [t][g][c] at t * 16 * G + g * 16 + c
// (G = k / 64), i.e. the 16 channels of a tile are contiguous per group.
//
// Rebuilding the int8 operand of one step for one lane (LiquidGEMM verdict
// page, pith_extraction.key_machinery, symmetric instance): per byte
//   v = u * s + (128 - 8 s)  stays in [16, 240] (no carry between bytes)
//   v XOR 0x80 read as int8 = (u - 8) * s = q * s in [-112, 112].
// The multiply-add runs on 16-bit halves (v_pk_mad_u16), two bytes per half.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Every binary32 product and sum below must round on its own: no contraction
// into fused multiply-adds (the build also passes -ffp-contract=off).
#pragma clang fp contract(off)

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;
constexpr int kNTile = 16;
constexpr int kChunkK = 128;
constexpr int kChunkBytes = 1024;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two binary32 values -> packed bf16 bits (lo in bits 0-15), one
// v_cvt_pk_bf16_f32: round to nearest even, subnormals kept, a NaN kept as the
// quiet NaN with the same sign and top payload bits ((u >> 16) | 0x40).  That is
// exactly u + 0x7fff + ((u >> 16) & 1), shifted right by 16, for every non-NaN
// bit pattern u; the instruction was compared with that integer form on all
// 2^32 inputs, NaNs included, with no difference.  As a vector conversion
// there is no branch per value (the integer form's NaN test compiled to one).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// round-half-even of v, saturated to [-lim, lim]; NaN gives 0.
__device__ __forceinline__ int sat_rne_code(float v, float lim) {
    float r = __builtin_rintf(v);
    r = __builtin_fminf(__builtin_fmaxf(r, -lim), lim);
    r = (v == v) ? r : 0.0f;
    return (int)r;
}

// 8 floats times inv -> 8 int8 codes rne(x * inv), little-endian in two words.
// With a finite inverse, |x * inv| <= 127 (1 + 2^-24)^2 < 127.5.  Adding
// 1.5 * 2^23 to the rounded product lands in [2^23, 2^24), where binary32
// spacing is 1, so the sum is 1.5 * 2^23 + rne(product) (ties to even, since
// 1.5 * 2^23 is even) and the low byte of its bits is the two's-complement
// code.  NaN products (0 * inf) give NaN sums whose low byte is 0.  An
// infinite inverse (amax below about 2^-121) takes the saturating path.
__device__ __forceinline__ u32x2 codes8(const float f[8], float inv) {
    uint32_t t[8];
    if (inv <= 3.40282347e38f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = f[i] * inv;
            t[i] = __float_as_uint(v + 12582912.0f);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = (uint32_t)sat_rne_code(f[i] * inv, 127.0f);
    }
    const uint32_t lo = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u) |
                        __builtin_amdgcn_perm(t[3], t[2], 0x04000c0cu);
    const uint32_t hi = __builtin_amdgcn_perm(t[5], t[4], 0x0c0c0400u) |
                        __builtin_amdgcn_perm(t[7], t[6], 0x04000c0cu);
    return u32x2{lo, hi};
}

// 8 bf16 (one 16-byte vector) -> 8 floats (exact).
__device__ __forceinline__ void bf16x8_to_f32(const u32x4 &v, float f[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ float absmax_f32x8(const float f[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
    return m;
}

// Activation block scale and inverse: s = amax / 127, inv = 127 / amax (0 if amax == 0).
__device__ __forceinline__ void act_scale_pair(float amax, float &s, float &inv) {
    s = amax / 127.0f;
    inv = (amax > 0.0f) ? (127.0f / amax) : 0.0f;
}

// Maximum of a non-negative 32-bit value over the 64 lanes of a wavefront with
// DPP row operations (quad swaps, half-row and row mirrors, then row broadcasts
// into rows 1-3); lane 63 ends with the total, which is returned to all lanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Maximum of a non-negative 32-bit value over aligned groups of LPB adjacent
// lanes (LPB a power of two up to 64), returned to every lane of the group:
// DPP quad swaps and half-row / row mirrors inside a row of 16 lanes (VALU
// operations, no LDS traffic), then lane swaps across rows.
template <int LPB>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if constexpr (LPB >= 2)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
    if constexpr (LPB >= 4)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
    if constexpr (LPB >= 8)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    if constexpr (LPB >= 16)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    if constexpr (LPB >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    if constexpr (LPB >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// Rebuild 4 int8 weights q*s from a word of 4 nibbles (one per byte, low bits).
// mul = s | s << 16, add = (128 - 8 s) * 0x01010101.
__device__ __forceinline__ int dequant4(uint32_t nib, uint32_t mul, uint32_t add) {
    v2u16 x = __builtin_bit_cast(v2u16, nib);
    v2u16 m = __builtin_bit_cast(v2u16, mul);
    v2u16 a = __builtin_bit_cast(v2u16, add);
    v2u16 r = x * m + a;
    return (int)(__builtin_bit_cast(uint32_t, r) ^ 0x80808080u);
}

__device__ __forceinline__ void scale_consts(uint32_t s, uint32_t &mul, uint32_t &add) {
    mul = s | (s << 16);
    uint32_t off = 128u - 8u * s;
    off |= off << 8;
    add = off | (off << 16);
}

// 16 packed weights of one K-step (two words) -> the 16-byte MFMA operand.
__device__ __forceinline__ v4i unpack_step(uint32_t p0, uint32_t p1, uint32_t mul,
                                           uint32_t add) {
    v4i r;
    r.x = dequant4(p0 & 0x0F0F0F0Fu, mul, add);
    r.y = dequant4((p0 >> 4) & 0x0F0F0F0Fu, mul, add);
    r.z = dequant4(p1 & 0x0F0F0F0Fu, mul, add);
    r.w = dequant4((p1 >> 4) & 0x0F0F0F0Fu, mul, add);
    return r;
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

typedef int v16i __attribute__((ext_vector_type(16)));

// v_mfma_i32_32x32x32_i8: lane l supplies A[row l % 32][k 16 (l / 32) .. +16] and
// B[k 16 (l / 32) .. +16][col l % 32]; result element r of lane l is
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ v16i mfma32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// global_load_lds_dwordx4: each lane copies 16 bytes from its own global address
// to LDS at lds_block + 16 * lane (lds_block must be the same for the whole
// wavefront).  Completion is tracked by vmcnt: wait before reading the block.
typedef __attribute__((address_space(1))) void *global_vptr;
typedef __attribute__((address_space(3))) void *lds_vptr;
__device__ __forceinline__ void global_to_lds16(const void *src, void *lds_block) {
    __builtin_amdgcn_global_load_lds((global_vptr)src, (lds_vptr)lds_block, 16, 0, 0);
}

// Raw (unstrided) buffer resource over [p, p + bytes).  A lane whose VGPR
// offset is at or past `bytes` reads zero and touches no memory; the scalar
// offset is added on top, so it must keep in-range lanes inside the buffer.
// Word 3 = 0x00020000 is the 32-bit data format in the gfx9 descriptor
// encoding, every other field zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// 16 bytes per lane straight into LDS at lds_block + 16 * lane (m0 = lds_block).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void *lds_block,
                                                int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds_block, 16, voff, soff, 0, 0);
}

// Byte offset of chunk j of n-tile t in the packed weights.
__device__ __forceinline__ int64_t packed_chunk_offset(int64_t t, int64_t j, int64_t k) {
    return t * (int64_t)kNTile * k / 2 + j * kChunkBytes;
}

// ------------------------------------------------------- weight formats --
// The GEMM kernels read three weight formats, all in 16-channel tiles and
// 128-wide K chunks with the same lane order (lane = c + 16 kq):
//   kW4Sym  layout V1 above; nibble u = q + 8; parameter per (tile, group,
//           channel) = uint8 group scale s; operand byte (u s + 128 - 8 s) ^ 0x80.
//   kW4Lqq  layout V1; nibble u = q_u4 in [0, 15]; parameter = uint16
//           s | a << 8 with a = 128 + group minimum; operand byte (u s + a) ^ 0x80
//           = u s + min (LiquidGEMM verdict page, pith_extraction.key_machinery,
//           in its own asymmetric form).
//   kW8     int8 weights: chunk j of tile t at t * 16 k + j * 2048; K step h at
//           + 1024 h, lane record of 16 bytes at + 16 lane (channel c,
//           k = 128 j + 64 h + 16 kq .. + 15); a trailing 64-wide chunk holds
//           step 0 only.  No parameter.
// Parameters are in kernel order [t][g][c] (element t * 16 G + g * 16 + c).
enum WFmt : int { kW4Sym = 0, kW4Lqq = 1, kW8 = 2 };

template <int WF> struct WRec { u32x4 r; };             // both K steps, 8 B each
template <> struct WRec<kW8> { u32x4 r0, r1; };         // 16 B per K step

template <int WF>
__device__ __forceinline__ uint32_t load_wparam(const uint8_t *p, int64_t idx) {
    if constexpr (WF == kW4Sym) return p[idx];
    else if constexpr (WF == kW4Lqq) return ((const uint16_t *)p)[idx];
    else return 0u;
}

// The aligned 32-bit word that holds parameter idx, and the parameter taken
// out of it.  A pipelined kernel keeps the word in flight across iterations:
// a byte or halfword load would come back as a narrow value that the compiler
// widens at the loop latch, which makes it wait for the load right there.
// The parameter array is 16-byte aligned and a multiple of 16 bytes long, so
// the word never leaves it.
template <int WF>
__device__ __forceinline__ uint32_t load_wparam_word(const uint8_t *p, int64_t idx) {
    if constexpr (WF == kW4Sym) return ((const uint32_t *)p)[idx >> 2];
    else if constexpr (WF == kW4Lqq) return ((const uint32_t *)p)[idx >> 1];
    else return 0u;
}
template <int WF>
__device__ __forceinline__ uint32_t wparam_from_word(uint32_t word, int64_t idx) {
    if constexpr (WF == kW4Sym) return (word >> (8 * (int)(idx & 3))) & 0xffu;
    else if constexpr (WF == kW4Lqq) return (word >> (16 * (int)(idx & 1))) & 0xffffu;
    else return 0u;
}

template <int WF>
__device__ __forceinline__ int64_t wchunk_offset(int64_t t, int64_t j, int64_t k) {
    if constexpr (WF == kW8) return t * (int64_t)kNTile * k + j * (2 * kChunkBytes);
    else return packed_chunk_offset(t, j, k);
}

// Full 128-wide chunk j of tile t, this lane's record (streamed: nontemporal).
template <int WF>
__device__ __forceinline__ WRec<WF> load_wrec(const uint8_t *w, int64_t t, int64_t j,
                                              int64_t k, int lane) {
    const uint8_t *base = w + wchunk_offset<WF>(t, j, k) + lane * 16;
    WRec<WF> rec;
    if constexpr (WF == kW8) {
        rec.r0 = __builtin_nontemporal_load((const u32x4 *)base);
        rec.r1 = __builtin_nontemporal_load((const u32x4 *)(base + kChunkBytes));
    } else {
        rec.r = __builtin_nontemporal_load((const u32x4 *)base);
    }
    return rec;
}

// Trailing 64-wide chunk j of tile t (step 0 only).
template <int WF>
__device__ __forceinline__ WRec<WF> load_wrec_half(const uint8_t *w, int64_t t, int64_t j,
                                                   int64_t k, int lane) {
    WRec<WF> rec;
    if constexpr (WF == kW8) {
        rec.r0 = *(const u32x4 *)(w + wchunk_offset<WF>(t, j, k) + lane * 16);
        rec.r1 = rec.r0;
    } else {
        const u32x2 h = *(const u32x2 *)(w + wchunk_offset<WF>(t, j, k) + lane * 8);
        rec.r = u32x4{h.x, h.y, 0u, 0u};
    }
    return rec;
}

// The 16-byte int8 operand of K step h (0 or 1) from a record and the step's
// group parameter.
template <int WF>
__device__ __forceinline__ v4i wrec_operand(const WRec<WF> &rec, int h, uint32_t param) {
    if constexpr (WF == kW8) {
        return __builtin_bit_cast(v4i, h ? rec.r1 : rec.r0);
    } else {
        uint32_t mul, add;
        if constexpr (WF == kW4Lqq) {
            const uint32_t s = param & 0xffu, a = param >> 8;
            mul = s | (s << 16);
            add = a * 0x01010101u;
        } else {
            scale_consts(param, mul, add);
        }
        return unpack_step(h ? rec.r.z : rec.r.x, h ? rec.r.w : rec.r.y, mul, add);
    }
}

// The rebuild constants straight from a parameter word (load_wparam_word):
// per-lane v_perm_b32 selectors pick this channel's parameter bytes.
//   kW4Sym  mul = s in bytes 0 and 2; add = 128 - 8 s in every byte, as one
//           packed 16-bit multiply-add per half: (128 - 8 s) * 257 =
//           32896 - 2056 s = s * (65536 - 2056) + 32896 (mod 2^16);
//   kW4Lqq  mul = s in bytes 0 and 2; add = a in every byte.
struct WParamSel { uint32_t mul, add; };
template <int WF>
__device__ __forceinline__ WParamSel wparam_selectors(int c) {
    const uint32_t bs = WF == kW4Lqq ? 2u * (c & 1) : (uint32_t)(c & 3);
    return WParamSel{bs | 0x0c00u | (bs << 16) | 0x0c000000u, (bs + 1u) * 0x01010101u};
}
template <int WF>
__device__ __forceinline__ void wparam_consts(uint32_t word, WParamSel sel, uint32_t &mul,
                                              uint32_t &add) {
    mul = __builtin_amdgcn_perm(0u, word, sel.mul);
    if constexpr (WF == kW4Lqq) add = __builtin_amdgcn_perm(0u, word, sel.add);
    else add = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, mul) *
                                              v2u16{(uint16_t)(65536 - 2056), (uint16_t)(65536 - 2056)} +
                                              v2u16{(uint16_t)32896, (uint16_t)32896});
}
template <int WF>
__device__ __forceinline__ v4i wrec_operand_ma(const WRec<WF> &rec, int h, uint32_t mul,
                                               uint32_t add) {
    if constexpr (WF == kW8) return __builtin_bit_cast(v4i, h ? rec.r1 : rec.r0);
    else return unpack_step(h ? rec.r.z : rec.r.x, h ? rec.r.w : rec.r.y, mul, add);
}

}  // namespace w4a8
