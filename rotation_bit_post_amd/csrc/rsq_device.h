// Device-side helpers shared by the kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8us __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Nearest-even rounding of a finite float to bfloat16 bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
// Split a float into bfloat16 hi + lo with hi + lo = f to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float f, uint16_t &hi, uint16_t &lo) {
    hi = f32_to_bf16(f);
    lo = f32_to_bf16(f - bf16_to_f32(hi));
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 (nearest even) in one word, low half first
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    v2bf p;
    p[0] = static_cast<__bf16>(a);
    p[1] = static_cast<__bf16>(b);
    uint32_t u;
    __builtin_memcpy(&u, &p, 4);
    return u;
}
__device__ __forceinline__ v2bf as_v2bf(uint32_t u) {
    v2bf p;
    __builtin_memcpy(&p, &u, 4);
    return p;
}

__device__ __forceinline__ v8bf as_v8bf(v4u x) {
    v8bf r;
    __builtin_memcpy(&r, &x, 16);
    return r;
}

// --------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}
__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// ---------------------------------------------------- quantisation kernels
// Code of a / s, for |a| <= qmax * s: the float32 quotient rounded to nearest,
// then to the nearest integer (ties to even), as in rint(a / s). The quotient
// starts as RN(a * inv_s) (inv_s = RN(1 / s)), within one ulp of a / s; one
// residual step r = a - y0 s (exact in an fma), y = RN(y0 + r inv_s) then
// gives RN(a / s) exactly (Markstein's theorem on fma-based division, IBM J.
// Res. Dev. 34(1), 1990). Adding 1.5 * 2^23 rounds y to an integer, ties to
// even, and leaves that integer in the low mantissa bits: the returned word's
// low 4 (or 3) bits are the two's complement code. s = 0 (inv_s = 0) gives 0.
__device__ __forceinline__ uint32_t quant_bits(float a, float s, float inv_s) {
    const float y0 = a * inv_s;
    const float r = fmaf(-y0, s, a);
    const float y = fmaf(r, inv_s, y0);
    return __float_as_uint(y + 12582912.0f);
}

// Eight 3-bit codes (the low 3 bits of u[e], two's complement) -> one word
// of fp4 e2m1 nibbles holding code / 2 (sign in bit 3, |code| in bits 0-1):
// code e < 4 in the high nibble of byte e, code e >= 4 in the low nibble of
// byte e - 4. |u| keeps u's low bit; its second bit flips where the sign and
// the low bit are both set (-1 -> 1, -3 -> 3, -2 -> 2).
__device__ __forceinline__ uint32_t fp4_word(const uint32_t u[8]) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= (u[e] & 7u) << (e < 4 ? 8 * e + 4 : 8 * (e - 4));
    const uint32_t sg = (w >> 2) & 0x11111111u;  // each nibble's sign, at its bit 0
    return ((w & 0x33333333u) ^ ((sg & w) << 1)) | (sg << 3);
}

// int3 packing without lane-dependent control flow. Lane group g (0..3) of a
// 32-code group holds codes 8g .. 8g+7 (code bits in the low 3 bits of u[e]),
// i.e. slots 2g (e < 4) and 2g + 1 (e >= 4), byte lane e % 4. Slots 2g and
// 2g+1 of g < 3 fill bits 5-7 and 2-4 of word g alone; slots 6 and 7 (g = 3)
// fill bits 0-1 of words 0 and 1 and bits 1 and 0 of word 2. own: this lane's
// contribution if g < 3; low[i]: its contribution to word i if g = 3.
__device__ __forceinline__ void int3_lane_parts(const uint32_t u[8], uint32_t &own, uint32_t low[3]) {
    own = 0;
    low[0] = low[1] = low[2] = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t lo = u[b] & 7u, hi = u[4 + b] & 7u;
        own |= (lo << (8 * b + 5)) | (hi << (8 * b + 2));
        low[0] |= (lo & 3u) << (8 * b);
        low[1] |= (hi & 3u) << (8 * b);
        low[2] |= ((lo >> 2) << (8 * b + 1)) | ((hi >> 2) << (8 * b));
    }
}

// ------------------------------------------------------- int8 unpacking
// int4: 16 codes (8 bytes, two words) -> four words of int8 holding 16 * code.
// Within each byte the nibble moves to bits 4-7, so the byte reads as 16 * code.
__device__ __forceinline__ v4i unpack_int4x16(uint32_t x0, uint32_t x1) {
    v4i r;
    r[0] = static_cast<int>((x0 << 4) & 0xF0F0F0F0u);
    r[1] = static_cast<int>(x0 & 0xF0F0F0F0u);
    r[2] = static_cast<int>((x1 << 4) & 0xF0F0F0F0u);
    r[3] = static_cast<int>(x1 & 0xF0F0F0F0u);
    return r;
}
// int3: one 32-code group (words w0, w1, w2) -> eight words of int8 holding
// 32 * code, slot j in word j (code 4j + b in byte b). half 0 gives slots 0-3,
// half 1 slots 4-7.
__device__ __forceinline__ v4i unpack_int3_half(uint32_t w0, uint32_t w1, uint32_t w2, int half) {
    v4i r;
    if (half == 0) {
        r[0] = static_cast<int>(w0 & 0xE0E0E0E0u);
        r[1] = static_cast<int>((w0 << 3) & 0xE0E0E0E0u);
        r[2] = static_cast<int>(w1 & 0xE0E0E0E0u);
        r[3] = static_cast<int>((w1 << 3) & 0xE0E0E0E0u);
    } else {
        r[0] = static_cast<int>(w2 & 0xE0E0E0E0u);
        r[1] = static_cast<int>((w2 << 3) & 0xE0E0E0E0u);
        r[2] = static_cast<int>(((w0 << 5) & 0x60606060u) | ((w2 << 6) & 0x80808080u));
        r[3] = static_cast<int>(((w1 << 5) & 0x60606060u) | ((w2 << 7) & 0x80808080u));
    }
    return r;
}

}  // namespace rsq
