// Row pieces held in registers (8 elements per lane and chunk) and the
// per-token RMSNorm + symmetric quantisation of one row by one wave.
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

// RMSNorm and per-token quantisation of one row of k elements by one wave
// (k <= 512 * CH): lane l holds the 8-element chunks l + 64 m. The same
// arithmetic as the standalone quantiser with its norm: float64 sum of
// squares (bf16 squares summed by 8 in float32 first), inv the float32
// rounding of 1 / sqrt(ss / k + eps), a = (x * inv) * w, s = max|a| / qmax,
// codes by the correctly rounded quotient of quant_bits. FMT: 4, 3 or kFp4.
template <typename T, int CH, int FMT>
__device__ __forceinline__ void quant_row_wave(const T *__restrict__ xr, int k, const float *__restrict__ norm_w,
                                               float eps, uint8_t *__restrict__ cr, float *__restrict__ scale,
                                               int lane) {
    const int nch = k / 8;
    Chunk8<T> v[CH];
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        if (lane + 64 * m < nch) v[m].load(xr + 8 * (lane + 64 * m));
        else v[m].zero();
    }
    double ss = 0.0;
    float am = 0.0f;
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        ss += v[m].sumsq();
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[m].get(e)));
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        ss += shfl_xor_f64(ss, off);
        am = wave_max_xor(am, off);
    }
    const float inv = static_cast<float>(1.0 / sqrt(ss / static_cast<double>(k) + static_cast<double>(eps)));
    float mval = am * inv;  // rounding is monotone: max|x * inv| = max|x| * inv
    if (norm_w != nullptr) {
        float a2 = 0.0f;
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            const int c = lane + 64 * m;
            if (c < nch)
#pragma unroll
                for (int e = 0; e < 8; ++e) a2 = fmaxf(a2, fabsf((v[m].get(e) * inv) * norm_w[8 * c + e]));
        }
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) a2 = wave_max_xor(a2, off);
        mval = a2;
    }
    constexpr int qmax = FMT == 4 ? 7 : 3;
    const float s = __fdiv_rn(mval, static_cast<float>(qmax));
    const float inv_s = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        const int c = lane + 64 * m;
        uint32_t u[8];
        if (norm_w != nullptr) {
            const int cc = c < nch ? c : nch - 1;
            const v4f w0 = *reinterpret_cast<const v4f *>(norm_w + 8 * cc);
            const v4f w1 = *reinterpret_cast<const v4f *>(norm_w + 8 * cc + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = quant_bits((v[m].get(e) * inv) * (e < 4 ? w0[e] : w1[e - 4]), s, inv_s);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = quant_bits(v[m].get(e) * inv, s, inv_s);
        }
        if constexpr (FMT == 4) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) word |= (u[e] & 0xFu) << (4 * e);
            if (c < nch) *reinterpret_cast<uint32_t *>(cr + 4 * c) = word;
        } else if constexpr (FMT == kFp4) {   // this chunk is word c % 4 of its 32-code group
            if (c < nch) *reinterpret_cast<uint32_t *>(cr + 4 * c) = fp4_word(u);
        } else {
            uint32_t own, low[3];
            int3_lane_parts(u, own, low);
            const int src = lane | 3;  // the lane holding slots 6 and 7 of this group
            const uint32_t l0 = __shfl(low[0], src, kWave), l1 = __shfl(low[1], src, kWave),
                           l2 = __shfl(low[2], src, kWave);
            const int q = lane & 3;
            const uint32_t word = own | (q == 0 ? l0 : (q == 1 ? l1 : l2));
            if (c < nch && q < 3) *reinterpret_cast<uint32_t *>(cr + 12 * (c >> 2) + 4 * q) = word;
        }
    }
    if (lane == 0) *scale = s;
}

}  // namespace rsq
