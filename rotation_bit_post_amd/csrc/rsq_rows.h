// Row pieces of the standalone quantiser held in registers (8 elements per lane and chunk).
#pragma once
#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

template <typename T> struct Chunk8;
template <> struct Chunk8<uint16_t> {  // bfloat16: 8 values in 16 bytes
    v4u raw;
    __device__ __forceinline__ void load(const uint16_t *p) { raw = *reinterpret_cast<const v4u *>(p); }
    __device__ __forceinline__ void zero() { raw = v4u{0, 0, 0, 0}; }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = raw[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    // squares of bf16 values are exact in float32; 8 of them are added in
    // float32, the chunks in float64
    __device__ __forceinline__ double sumsq() const {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) s = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(raw[q]), as_v2bf(raw[q]), s, false);
        return static_cast<double>(s);
    }
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(raw)); }
};
template <> struct Chunk8<float> {
    v4f a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const v4f *>(p);
        b = *reinterpret_cast<const v4f *>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = v4f{0, 0, 0, 0}; b = a; }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
    __device__ __forceinline__ double sumsq() const {  // float64 products and adds
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fma(static_cast<double>(get(e)), static_cast<double>(get(e)), s);
        return s;
    }
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(a), "+v"(b)); }
};

}  // namespace rsq
