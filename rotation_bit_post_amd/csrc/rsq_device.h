// Device-side helpers shared by the kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsq {

typedef int v4i __attribute__((ext_vector_type(4)));
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
// rint(a / s) with the float32 quotient rounded to nearest (ties to even),
// computed as a * inv_s (inv_s = 1/s correctly rounded). The product is within
// 2^-23 relative of a / s, so it can differ in rounding only when a / s is
// within a few ulps of a half-integer; those rare cases take the exact division.
__device__ __forceinline__ int quant_code(float a, float s, float inv_s, int qmax) {
    float y = a * inv_s;
    float ay = fabsf(y);
    float frac = ay - floorf(ay);
    float q;
    if (fabsf(frac - 0.5f) < 4.0e-6f) {
        q = rintf(__fdiv_rn(a, s));
    } else {
        q = rintf(y);
    }
    q = fminf(fmaxf(q, -static_cast<float>(qmax)), static_cast<float>(qmax));
    return static_cast<int>(q);
}

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

// Pack 8 int4 codes (code e at nibble e) into one 32-bit word: byte j = c[2j] | c[2j+1] << 4.
__device__ __forceinline__ uint32_t pack_int4x8(const int c[8]) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= (static_cast<uint32_t>(c[e]) & 0xFu) << (4 * e);
    return w;
}

// Contribution of 8 consecutive int3 codes (codes 8q..8q+7 of a 32-code group)
// to the group's three words. OR-ing the contributions of q = 0..3 gives the group.
__device__ __forceinline__ void int3_part(const int c[8], int q, uint32_t &w0, uint32_t &w1, uint32_t &w2) {
    w0 = w1 = w2 = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t u = static_cast<uint32_t>(c[e]) & 7u;
        const int slot = 2 * q + (e >> 2);
        const int b = e & 3;
        const int base = 8 * b;
        if (slot < 6) {
            const int shift = base + ((slot & 1) ? 2 : 5);
            const uint32_t bits = u << shift;
            if ((slot >> 1) == 0) w0 |= bits; else if ((slot >> 1) == 1) w1 |= bits; else w2 |= bits;
        } else if (slot == 6) {
            w0 |= (u & 3u) << base;
            w2 |= ((u >> 2) & 1u) << (base + 1);
        } else {
            w1 |= (u & 3u) << base;
            w2 |= ((u >> 2) & 1u) << base;
        }
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
