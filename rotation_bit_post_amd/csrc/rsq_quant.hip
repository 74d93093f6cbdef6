// Per-token symmetric activation quantisation with optional RMSNorm.
//
// WPR waves (1 or 4) own one row and keep it in registers across the
// three steps (statistics, scale, quantise + pack), so the row is read from
// HBM once; a 256-thread workgroup holds 4 / WPR rows. Lane l of wave s of a
// row owns the 8-element chunks s*64 + l + 64*WPR*m, so a wave's loads are
// contiguous. Statistics reduce in a fixed order (lane tree, then the row's
// waves through LDS), so the result does not depend on scheduling. The four
// chunks of a 32-code int3 group sit in four neighbouring lanes.
#include "rsq_device.h"
#include "rsq_internal.h"
#include "rsq_rows.h"

namespace rsq {

namespace {

constexpr int kThreads = 256;

// CH: chunks per lane (compile time); WPR: waves per row; FMT: code format
// (4, 3 or kFp4), a template parameter so that no instance carries the
// branches of the others.
template <typename T, int CH, int WPR, int FMT>
__global__ __launch_bounds__(kThreads) void quant_kernel(const T *__restrict__ x, int64_t n, int k, int64_t ld_x,
                                                        int norm, const float *__restrict__ norm_w, float eps,
                                                        uint8_t *__restrict__ codes, float *__restrict__ scales) {
    constexpr int RPB = 4 / WPR;  // rows per workgroup
    __shared__ double lss[4];
    __shared__ float lam[4], lwm[4];
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int rw = w / WPR, sub = w % WPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + rw;
    const bool rvalid = row < n;
    const int nch = k / 8;
    const T *xr = x + (rvalid ? row : n - 1) * ld_x;
    auto chunk = [&](int m) { return sub * 64 + lane + 64 * WPR * m; };

    Chunk8<T> v[CH];
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        if (chunk(m) < nch) v[m].load(xr + 8 * chunk(m));
        else v[m].zero();
    }

    // statistics: sum of squares and max |x|
    double ss = 0.0;
    float am = 0.0f;
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        if (norm) ss += v[m].sumsq();
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[m].get(e)));
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        ss += shfl_xor_f64(ss, off);
        am = wave_max_xor(am, off);
    }
    if constexpr (WPR > 1) {
        if (lane == 0) { lss[w] = ss; lam[w] = am; }
        __syncthreads();
        ss = 0.0;
        am = 0.0f;
#pragma unroll
        for (int i = 0; i < WPR; ++i) { ss += lss[rw * WPR + i]; am = fmaxf(am, lam[rw * WPR + i]); }
    }

    float inv = 1.0f;
    float mval = am;
    if (norm) {
        inv = static_cast<float>(1.0 / sqrt(ss / static_cast<double>(k) + static_cast<double>(eps)));
        if (norm_w == nullptr) {
            mval = am * inv;  // rounding is monotone: max|x * inv| = max|x| * inv
        } else {
            float a2 = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                const int c = chunk(m);
                if (c < nch)
#pragma unroll
                    for (int e = 0; e < 8; ++e) a2 = fmaxf(a2, fabsf((v[m].get(e) * inv) * norm_w[8 * c + e]));
            }
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) a2 = wave_max_xor(a2, off);
            if constexpr (WPR > 1) {
                if (lane == 0) lwm[w] = a2;
                __syncthreads();
                a2 = 0.0f;
#pragma unroll
                for (int i = 0; i < WPR; ++i) a2 = fmaxf(a2, lwm[rw * WPR + i]);
            }
            mval = a2;
        }
    }
#pragma unroll
    for (int m = 0; m < CH; ++m) v[m].opaque();
    constexpr int qmax = FMT == 4 ? 7 : 3;
    const float s = __fdiv_rn(mval, static_cast<float>(qmax));
    const float inv_s = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
    const size_t rowb = FMT == 3 ? static_cast<size_t>(k) * 3 / 8 : static_cast<size_t>(k) / 2;
    uint8_t *cr = codes + (rvalid ? row : 0) * rowb;

    // quantise + pack; a = x (no norm), x * inv, or (x * inv) * w
    auto quant_chunk = [&](int m, bool nrm, const float *wts) {
        const int c = chunk(m);
        uint32_t u[8];
        if (wts != nullptr) {
            const int cc = c < nch ? c : nch - 1;
            const v4f w0 = *reinterpret_cast<const v4f *>(wts + 8 * cc);
            const v4f w1 = *reinterpret_cast<const v4f *>(wts + 8 * cc + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = quant_bits((v[m].get(e) * inv) * (e < 4 ? w0[e] : w1[e - 4]), s, inv_s);
        } else if (nrm) {
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = quant_bits(v[m].get(e) * inv, s, inv_s);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = quant_bits(v[m].get(e), s, inv_s);
        }
        if constexpr (FMT == 4) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) word |= (u[e] & 0xFu) << (4 * e);
            if (rvalid && c < nch) *reinterpret_cast<uint32_t *>(cr + 4 * c) = word;
        } else if constexpr (FMT == kFp4) {   // this chunk is word c % 4 of its 32-code group
            if (rvalid && c < nch) *reinterpret_cast<uint32_t *>(cr + 4 * c) = fp4_word(u);
        } else {
            uint32_t own, low[3];
            int3_lane_parts(u, own, low);
            const int src = lane | 3;  // the lane holding slots 6 and 7 of this group
            const uint32_t l0 = __shfl(low[0], src, kWave), l1 = __shfl(low[1], src, kWave),
                           l2 = __shfl(low[2], src, kWave);
            const int q = lane & 3;
            const uint32_t word = own | (q == 0 ? l0 : (q == 1 ? l1 : l2));
            if (rvalid && c < nch && q < 3) *reinterpret_cast<uint32_t *>(cr + 12 * (c >> 2) + 4 * q) = word;
        }
    };
    if (norm && norm_w != nullptr) {
#pragma unroll
        for (int m = 0; m < CH; ++m) quant_chunk(m, true, norm_w);
    } else if (norm) {
#pragma unroll
        for (int m = 0; m < CH; ++m) quant_chunk(m, true, nullptr);
    } else {
#pragma unroll
        for (int m = 0; m < CH; ++m) quant_chunk(m, false, nullptr);
    }
    if (rvalid && sub == 0 && lane == 0) scales[row] = s;
}

template <typename T, int CH, int WPR>
hipError_t launch_t(const void *x, int64_t n, int k, int64_t ld_x, bool norm, const float *norm_w, float eps,
                    int bits, uint8_t *codes, float *scales, hipStream_t s) {
    constexpr int RPB = 4 / WPR;
    if (!grid_fits((n + RPB - 1) / RPB, kThreads)) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>((n + RPB - 1) / RPB));
    const T *xt = static_cast<const T *>(x);
    if (bits == 4)
        hipLaunchKernelGGL((quant_kernel<T, CH, WPR, 4>), grid, dim3(kThreads), 0, s, xt, n, k, ld_x, norm ? 1 : 0,
                           norm_w, eps, codes, scales);
    else if (bits == kFp4)
        hipLaunchKernelGGL((quant_kernel<T, CH, WPR, kFp4>), grid, dim3(kThreads), 0, s, xt, n, k, ld_x, norm ? 1 : 0,
                           norm_w, eps, codes, scales);
    else
        hipLaunchKernelGGL((quant_kernel<T, CH, WPR, 3>), grid, dim3(kThreads), 0, s, xt, n, k, ld_x, norm ? 1 : 0,
                           norm_w, eps, codes, scales);
    return hipGetLastError();
}

// Rows up to 512 elements: one wave per row, one chunk per lane. Longer rows:
// four waves per row, each lane with the fewest chunks that cover the row
// (ceil(k / 2048)). Measured on MI355X against the earlier choice of one wave
// up to 4096 elements and chunk counts rounded up to a power of two (cold
// inputs, outputs byte-identical): 2048 x 4096 6.8 -> 6.3 us, 2048 x 11008
// 13.7 -> 13.2 us, 4096 x 8192 16.8 -> 16.2 us, 4096 x 28672 58.5 -> 52.9 us.
template <typename T>
hipError_t launch_w(const void *x, int64_t n, int k, int64_t ld_x, bool norm, const float *norm_w, float eps,
                    int bits, uint8_t *codes, float *scales, hipStream_t s) {
    const int nch = k / 8;
    if (nch <= 64) return launch_t<T, 1, 1>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    switch ((nch + 255) / 256) {
        case 1: return launch_t<T, 1, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 2: return launch_t<T, 2, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 3: return launch_t<T, 3, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 4: return launch_t<T, 4, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 5: return launch_t<T, 5, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 6: return launch_t<T, 6, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 7: return launch_t<T, 7, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 8: return launch_t<T, 8, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 9: return launch_t<T, 9, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 10: return launch_t<T, 10, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 11: return launch_t<T, 11, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 12: return launch_t<T, 12, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 13: return launch_t<T, 13, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 14: return launch_t<T, 14, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 15: return launch_t<T, 15, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        case 16: return launch_t<T, 16, 4>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quant(const void *x, int x_dtype, int64_t n, int k, int64_t ld_x, bool norm,
                        const float *norm_w, float eps, int bits, uint8_t *codes, float *scales,
                        hipStream_t s) {
    if (x_dtype == 1) return launch_w<uint16_t>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
    return launch_w<float>(x, n, k, ld_x, norm, norm_w, eps, bits, codes, scales, s);
}

}  // namespace rsq
