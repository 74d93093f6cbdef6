// Per-token symmetric activation quantisation with optional RMSNorm.
//
// One 256-thread workgroup per row: thread t owns 8-element chunks
// t, t + 256, ... of the row and keeps them in registers across the three
// steps (statistics, scale, quantise + pack), so the row is read from HBM
// once. Statistics reduce in a fixed order (lane tree, then waves), so the
// result does not depend on scheduling. Chunks 4i..4i+3 (one 32-code group)
// sit in 4 neighbouring lanes, which lets the int3 words be assembled with
// two lane exchanges.
#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

namespace {

constexpr int kThreads = 256;

template <typename T> struct Chunk8;
template <> struct Chunk8<uint16_t> {
    v4u raw;
    __device__ __forceinline__ void load(const uint16_t *p) { raw = *reinterpret_cast<const v4u *>(p); }
    __device__ __forceinline__ void zero() { raw = v4u{0, 0, 0, 0}; }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = raw[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};
template <> struct Chunk8<float> {
    v4f a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const v4f *>(p);
        b = *reinterpret_cast<const v4f *>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = v4f{0, 0, 0, 0}; b = a; }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// CH: maximum chunks per thread (compile time); the row has k / 8 chunks.
template <typename T, int CH>
__global__ __launch_bounds__(kThreads) void quant_kernel(const T *__restrict__ x, int64_t n, int k, int64_t ld_x,
                                                        int norm, const float *__restrict__ norm_w, float eps,
                                                        int bits, uint8_t *__restrict__ codes,
                                                        float *__restrict__ scales) {
    __shared__ double ssq[kThreads / kWave];
    __shared__ float amx[kThreads / kWave];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nch = k / 8;
    const T *xr = x + row * ld_x;

    Chunk8<T> v[CH];
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        const int c = tid + kThreads * m;
        if (c < nch) v[m].load(xr + 8 * c);
        else v[m].zero();
    }

    // statistics: sum of squares (float64) and max |x|
    double ss = 0.0;
    float am = 0.0f;
#pragma unroll
    for (int m = 0; m < CH; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = v[m].get(e);
            ss = fma(static_cast<double>(xv), static_cast<double>(xv), ss);
            am = fmaxf(am, fabsf(xv));
        }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        ss += shfl_xor_f64(ss, off);
        am = wave_max_xor(am, off);
    }
    if (lane == 0) { ssq[wv] = ss; amx[wv] = am; }
    __syncthreads();
    double tot = 0.0;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) { tot += ssq[i]; amax = fmaxf(amax, amx[i]); }

    float inv = 1.0f;
    float mval = amax;
    if (norm) {
        inv = static_cast<float>(1.0 / sqrt(tot / static_cast<double>(k) + static_cast<double>(eps)));
        if (norm_w == nullptr) {
            mval = amax * inv;  // rounding is monotone: max|x * inv| = max|x| * inv
        } else {
            float a2 = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                const int c = tid + kThreads * m;
                if (c < nch)
#pragma unroll
                    for (int e = 0; e < 8; ++e) a2 = fmaxf(a2, fabsf((v[m].get(e) * inv) * norm_w[8 * c + e]));
            }
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) a2 = wave_max_xor(a2, off);
            __syncthreads();
            if (lane == 0) amx[wv] = a2;
            __syncthreads();
            mval = 0.0f;
#pragma unroll
            for (int i = 0; i < kThreads / kWave; ++i) mval = fmaxf(mval, amx[i]);
        }
    }
    const int qmax = (1 << (bits - 1)) - 1;
    const float s = __fdiv_rn(mval, static_cast<float>(qmax));
    const float inv_s = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
    const size_t rowb = bits == 4 ? static_cast<size_t>(k) / 2 : static_cast<size_t>(k) * 3 / 8;
    uint8_t *cr = codes + row * rowb;

#pragma unroll
    for (int m = 0; m < CH; ++m) {
        const int c = tid + kThreads * m;
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = v[m].get(e);
            if (norm) {
                a *= inv;
                if (norm_w != nullptr && c < nch) a *= norm_w[8 * c + e];
            }
            q[e] = s > 0.0f ? quant_code(a, s, inv_s, qmax) : 0;
        }
        if (bits == 4) {
            if (c < nch) *reinterpret_cast<uint32_t *>(cr + 4 * c) = pack_int4x8(q);
        } else if (kThreads * m < nch) {  // whole 32-code groups are in or out together
            uint32_t w0, w1, w2;
            const int qpos = c & 3;
            int3_part(q, qpos, w0, w1, w2);
            w0 |= __shfl_xor(w0, 1, kWave); w0 |= __shfl_xor(w0, 2, kWave);
            w1 |= __shfl_xor(w1, 1, kWave); w1 |= __shfl_xor(w1, 2, kWave);
            w2 |= __shfl_xor(w2, 1, kWave); w2 |= __shfl_xor(w2, 2, kWave);
            if (c < nch && qpos < 3)
                *reinterpret_cast<uint32_t *>(cr + 12 * (c >> 2) + 4 * qpos) = qpos == 0 ? w0 : (qpos == 1 ? w1 : w2);
        }
    }
    if (tid == 0) scales[row] = s;
}

template <typename T, int CH>
hipError_t launch_t(const void *x, int64_t n, int k, int64_t ld_x, bool norm, const float *norm_w, float eps,
                    int bits, uint8_t *codes, float *scales, hipStream_t s) {
    hipLaunchKernelGGL((quant_kernel<T, CH>), dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, s,
                       static_cast<const T *>(x), n, k, ld_x, norm ? 1 : 0, norm_w, eps, bits, codes, scales);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_ch(const void *x, int64_t n, int k, int64_t ld_x, bool norm, const float *norm_w, float eps,
                     int bits, uint8_t *codes, float *scales, hipStream_t s) {
    const int need = (k / 8 + kThreads - 1) / kThreads;
    if (need <= 1) return launch_t<T, 1>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    if (need <= 2) return launch_t<T, 2>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    if (need <= 4) return launch_t<T, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    if (need <= 8) return launch_t<T, 8>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    if (need <= 16) return launch_t<T, 16>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quant(const void *x, int x_dtype, int64_t n, int k, int64_t ld_x, bool norm,
                        const float *norm_w, float eps, int bits, uint8_t *codes, float *scales,
                        hipStream_t s) {
    if (x_dtype == 1) return launch_ch<uint16_t>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    return launch_ch<float>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
}

}  // namespace rsq
