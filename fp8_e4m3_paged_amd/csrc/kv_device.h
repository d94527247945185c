// Device-side helpers shared by the kernels: vector types, tile layouts and
// the gfx950 FP8 conversions. gfx950 only; no other target is built.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp8 {

constexpr int kPage = 16;          // tokens per page
constexpr int kDim = 128;          // head_dim
constexpr int kTileFp8 = kPage * kDim;        // 2048 bytes
constexpr int kTileBf16 = kPage * kDim * 2;   // 4096 bytes

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Byte offset of element (token t, dim d) inside one (page, head) tile.
// These are the layouts documented in kvfp8.h; the append kernels write
// through them and the attention kernel's loads are their inverse.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int off_k_fp8(int t, int d) {
    return 1024 * ((d % 32) / 16) + 256 * (d / 32) + 16 * t + (d % 16);
}
__host__ __device__ __forceinline__ int off_v_fp8(int t, int d) {
    return 1024 * (d / 64) + 256 * (t / 4) + 16 * (d % 16) + 4 * ((d / 16) % 4) + (t % 4);
}
__host__ __device__ __forceinline__ int off_k_bf16(int t, int d) {
    return 1024 * ((d % 32) / 8) + 256 * (d / 32) + 16 * t + 2 * (d % 8);
}
__host__ __device__ __forceinline__ int off_v_bf16(int t, int d) {
    return 1024 * (d / 32) + 256 * (t / 4) + 16 * (d % 16) + 8 * ((d / 16) % 2) + 2 * (t % 4);
}

// ---------------------------------------------------------------------------
// FP8 e4m3 (OCP) conversions on gfx950.
// ---------------------------------------------------------------------------

// Encode two floats already divided by the scale. Finite values and
// infinities are clamped to +-448 first, so the hardware's round-to-nearest-
// even conversion never sees an overflow; NaN gets the NaN code with its sign.
__device__ __forceinline__ uint32_t sat_e4m3_byte_fixup(float y, uint32_t code) {
    if (y != y) return (__float_as_uint(y) >> 24 & 0x80u) | 0x7Fu;
    return code;
}

__device__ __forceinline__ float clamp448(float y) {
    // fminf/fmaxf would turn NaN into +-448; NaN is fixed up after the convert.
    return (y != y) ? 0.0f : fminf(fmaxf(y, -448.0f), 448.0f);
}

// x / s rounded to fp32 with round-to-odd. The correctly rounded quotient y
// alone is not enough: with bf16 x and s = amax / 448 the exact quotient is
// often a hair away from an e4m3 midpoint, y then lands exactly on the
// midpoint and the final round-half-even picks the wrong side. The fma
// remainder r = x - y*s is exact, so the sign of r/s says on which side of y
// the exact quotient lies; truncating toward zero and forcing the last bit to
// 1 when inexact gives round-to-odd, and a round-to-odd value with >= 4 + 2
// significand bits rounds to E4M3 exactly as the exact quotient would.
// Written with selects only (no early returns), so the encoder runs without
// divergent branches; zero, infinite and NaN quotients and exact ones pass
// through unchanged.
__device__ __forceinline__ float div_round_odd(float x, float s) {
    const float y = x / s;                       // correctly rounded (IEEE) division
    const float r = fmaf(-y, s, x);              // exact remainder (finite y)
    const bool inexact = fabsf(y) < INFINITY && y != 0.0f && r != 0.0f;
    const bool toward_zero = ((r < 0.0f) != (s < 0.0f)) != (y < 0.0f);
    uint32_t u = __float_as_uint(y);
    u -= (inexact && toward_zero) ? 1u : 0u;     // |y| - 1 ulp: the truncated quotient
    u |= inexact ? 1u : 0u;
    return __uint_as_float(u);
}

// Four floats (already x / s, round-to-odd) -> four e4m3 codes, little-endian.
__device__ __forceinline__ uint32_t encode4_e4m3(float y0, float y1, float y2, float y3) {
    uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y0), clamp448(y1), 0u, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y2), clamp448(y3), pk, true);
    uint32_t b0 = sat_e4m3_byte_fixup(y0, pk & 0xFFu);
    uint32_t b1 = sat_e4m3_byte_fixup(y1, (pk >> 8) & 0xFFu);
    uint32_t b2 = sat_e4m3_byte_fixup(y2, (pk >> 16) & 0xFFu);
    uint32_t b3 = sat_e4m3_byte_fixup(y3, (pk >> 24) & 0xFFu);
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Decode the 4 e4m3 codes of one dword into 4 bf16 (exact: 4 significant
// bits fit bf16's 8). Scale operand 1.0 keeps the conversion a pure decode.
__device__ __forceinline__ void decode4_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

// Decode the 4 e4m3 codes of one dword into 4 f16 (exact: every e4m3 value,
// subnormals included, is an f16 normal).
__device__ __forceinline__ void decode4_f16(uint32_t w, f16x2& lo, f16x2& hi) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Store 4 consecutive dims d..d+3 (bf16 bits in raw) of one token into slot
// `slot` of a (page, head) tile: FP8 quantizes with the scale s first. K keeps
// the 4 dims contiguous (one dword / one 8-byte store); V is token-minor, so
// its 4 dims land 16 bytes apart. Both append paths use this one routine.
template <bool FP8>
__device__ __forceinline__ void store_token_quad(bool is_v, u32x2 raw, float s, uint8_t* tile_base,
                                        int slot, int d) {
    if constexpr (FP8) {
        const float y0 = div_round_odd(bf16_bits_to_float(raw.x & 0xFFFF), s);
        const float y1 = div_round_odd(bf16_bits_to_float(raw.x >> 16), s);
        const float y2 = div_round_odd(bf16_bits_to_float(raw.y & 0xFFFF), s);
        const float y3 = div_round_odd(bf16_bits_to_float(raw.y >> 16), s);
        const uint32_t codes = encode4_e4m3(y0, y1, y2, y3);
        if (!is_v) {
            *reinterpret_cast<uint32_t*>(tile_base + off_k_fp8(slot, d)) = codes;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) tile_base[off_v_fp8(slot, d + i)] = (codes >> (8 * i)) & 0xFF;
        }
    } else {
        if (!is_v) {
            *reinterpret_cast<u32x2*>(tile_base + off_k_bf16(slot, d)) = raw;
        } else {
            const uint16_t h[4] = {static_cast<uint16_t>(raw.x & 0xFFFF),
                                   static_cast<uint16_t>(raw.x >> 16),
                                   static_cast<uint16_t>(raw.y & 0xFFFF),
                                   static_cast<uint16_t>(raw.y >> 16)};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint16_t*>(tile_base + off_v_bf16(slot, d + i)) = h[i];
        }
    }
}

}  // namespace kvfp8
