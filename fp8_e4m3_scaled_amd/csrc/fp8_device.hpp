// Device helpers for OCP E4M3 ("e4m3fn") on gfx950.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvf8 {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Saturating round-half-even E4M3 of two fp32 values, packed into the low
// 16 bits (a in bits 0-7, b in bits 8-15).  The page's encoder [P2,
// ggml_fp32_to_f8_e4m3] maps NaN to sign|0x7F and +-Inf / |x| >= 448 to
// sign|0x7E; the hardware convert rounds half-even but does not saturate
// Inf, so values are clamped to +-448 first (med3 keeps in-range values and
// the sign of zero), and NaN is rebuilt from its own sign bit.
__device__ __forceinline__ uint32_t encode2(float a, float b) {
    const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (__builtin_isnan(a)) r = (r & 0xFF00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
    if (__builtin_isnan(b)) r = (r & 0x00FFu) | ((((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu) << 8);
    return r;
}

// Four fp32 values -> four codes in one dword (a in the lowest byte).
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
    return encode2(a, b) | (encode2(c, d) << 16);
}

// encode4 for values known not to be NaN (saturation still applies).
__device__ __forceinline__ uint32_t encode4_finite(float a, float b, float c, float d) {
    const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    const float cc = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    const float cd = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, lo, true);
}

// True when any of the four codes in w is NaN (low seven bits all ones).
__device__ __forceinline__ bool has_nan4(uint32_t w) {
    return (((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) != 0u;
}

// Bit 7 of every byte of w that holds an E4M3 NaN code (0x7F or 0xFF).
__device__ __forceinline__ uint32_t e4m3_nan_bytes(uint32_t w) {
    return ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// Bit 15 of every 16-bit half of w that holds a bf16 infinity or NaN
// (exponent field all ones).
__device__ __forceinline__ uint32_t bf16_nonfinite_halves(uint32_t w) {
    return ((w & 0x7F807F80u) + 0x00800080u) & 0x80008000u;
}

// Class bits of the non-finite halves n (bf16_nonfinite_halves) of w: 1 for
// a NaN, 2 for +Inf, 4 for -Inf.
__device__ __forceinline__ uint32_t bf16_class_bits(uint32_t w, uint32_t n) {
    uint32_t c = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!((n >> (16 * h + 15)) & 1u)) continue;
        const uint32_t v = (w >> (16 * h)) & 0xFFFFu;
        c |= (v & 0x7Fu) ? 1u : (v & 0x8000u) ? 4u : 2u;
    }
    return c;
}

// What non-finite values of the classes c (bf16_class_bits, ORed) add to a sum
// of products with positive weights: NaN if any is NaN or both infinities
// occur, else an infinity of the one sign, else 0.
__device__ __forceinline__ float nonfinite_from_bits(uint32_t c) {
    if (c & 1u) return __builtin_nanf("");
    float t = 0.0f;
    if (c & 2u) t = __builtin_inff();
    if (c & 4u) t = t - __builtin_inff();          // +Inf - Inf is NaN
    return t;
}

// Multiply a bf16 value by the reciprocal scale; a NaN input keeps its own
// sign (the sign of a NaN produced by an arithmetic operation is not fixed
// by IEEE 754).
__device__ __forceinline__ float scaled(uint32_t bits16, float inv) {
    const float x = bf16_to_f32(bits16);
    return __builtin_isnan(x) ? x : x * inv;
}

// Codes -> exact bf16 / f16 pairs (every E4M3 value is exact in both).
// HI selects bytes 2-3 of the dword instead of bytes 0-1.
template <bool HI>
__device__ __forceinline__ bf16x2 codes_to_bf16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}
template <bool HI>
__device__ __forceinline__ f16x2 codes_to_f16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
template <bool HI>
__device__ __forceinline__ f32x2 codes_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

}  // namespace kvf8
