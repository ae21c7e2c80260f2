// Element arithmetic shared by the block quantizers of libw8a8 (not installed).
//
// q = rint(fl32(x / s)) ties to even, for |x| <= 127 s: with r = fl32(1/s)
// computed once per block, q0 = x*r, e = fma(-q0, s, x) (the exact remainder)
// and q1 = fma(e, r, q0) equal the correctly rounded fl32(x/s) (Markstein's
// correction; checked exhaustively against correctly rounded division for
// every pair of bf16 values 0 < x <= a with s = fl32(a/127)).  Scales below
// 2^-60 need x and s both multiplied by 2^64 first (exact) so that 1/s stays
// finite and the remainder stays normal.  q1 + 1.5*2^23 rounds q1 to the
// nearest-even integer, whose low 8 mantissa bits are q in two's complement
// (|q1| <= 127, so no clamp is ever active).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kTinyScale = 0x1p-60f;      // scales below this take the 2^64 prescale
constexpr float kPrescale = 0x1p64f;

__device__ __forceinline__ uint32_t code_byte(float x, float ss, float r) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, ss, x);
    const float q1 = __builtin_fmaf(e, r, q0);
    return __float_as_uint(q1 + kRoundMagic) & 0xFFu;
}

// Four codes from two words of packed bf16 (lo holds elements 0, 1 and hi
// elements 2, 3, little endian); kScaled multiplies each value by f first.
template <bool kScaled>
__device__ __forceinline__ uint32_t code_word(uint32_t lo, uint32_t hi, float f, float ss, float r) {
    float v0 = __uint_as_float(lo << 16), v1 = __uint_as_float(lo & 0xFFFF0000u);
    float v2 = __uint_as_float(hi << 16), v3 = __uint_as_float(hi & 0xFFFF0000u);
    if (kScaled) {
        v0 *= f;
        v1 *= f;
        v2 *= f;
        v3 *= f;
    }
    return code_byte(v0, ss, r) | (code_byte(v1, ss, r) << 8) | (code_byte(v2, ss, r) << 16) |
           (code_byte(v3, ss, r) << 24);
}

// Eight codes of one 16-byte chunk of bf16.
template <bool kScaled>
__device__ __forceinline__ u32x2 code_chunk(u32x4 w, float f, float ss, float r) {
    return u32x2{code_word<kScaled>(w.x, w.y, f, ss, r), code_word<kScaled>(w.z, w.w, f, ss, r)};
}

// Largest 15-bit magnitude over a chunk of bf16 (for non-negative floats the
// bit order is the value order).
__device__ __forceinline__ uint32_t chunk_absmax_bits(u32x4 w) {
    const uint32_t a = max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu);
    const uint32_t b = max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu);
    const uint32_t c = max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu);
    const uint32_t d = max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu);
    return max(max(a, b), max(c, d));
}

}  // namespace w8a8
