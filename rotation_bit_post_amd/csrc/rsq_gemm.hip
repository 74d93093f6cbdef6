// Quantised linear: int4 / int3 codes on the int8 matrix cores.
//
//   acc[t, j] = sum_k a[t, k] w[j, k]            (int32, exact)
//   y[t, j]   = (float(acc) * s_a[t]) * s_w[j]
//
// Packed tiles go from HBM/L2 to LDS unchanged (double buffered, one barrier
// per 128-code k step) and are widened to int8 in registers right before
// v_mfma_i32_32x32x32_i8. Widening only moves each code's bits to the top of
// its byte, so the matrix core multiplies 16*a by 16*w (int4) or 32*a by
// 32*w (int3); the epilogue shifts the exact accumulator back. With codes in
// [-7, 7] and K <= 28672 the scaled sum stays below 2^29. The k order inside
// a 32-code step is permuted the same way for both operands, which leaves the
// dot products unchanged.
//
// Matrix-core roles: A = activations (rows = tokens), B = weights (columns =
// output channels), so each store instruction writes 32 consecutive channels
// of a token row.
#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

namespace {

constexpr int kBK = 128;  // codes per k step

template <int BITS> struct Fmt;
template <> struct Fmt<4> {
    static constexpr int kRowB = 64;     // packed bytes of 128 codes
    static constexpr int kStride = 72;   // LDS row stride (bank-conflict-free 8-byte reads)
    static constexpr int kShift = 8;     // (16 a)(16 w) = 256 a w
};
template <> struct Fmt<3> {
    static constexpr int kRowB = 48;
    static constexpr int kStride = 52;
    static constexpr int kShift = 10;    // (32 a)(32 w) = 1024 a w
};

template <typename YT> __device__ __forceinline__ YT to_out(float v);
template <> __device__ __forceinline__ float to_out<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t to_out<uint16_t>(float v) { return f32_to_bf16(v); }

// Operand for one 32-code step s of a row held in LDS (lane half h = lane / 32).
template <int BITS>
__device__ __forceinline__ v4i lds_operand(const uint8_t *rowp, int s, int h) {
    if constexpr (BITS == 4) {
        const v2u x = *reinterpret_cast<const v2u *>(rowp + 16 * s + 8 * h);
        return unpack_int4x16(x[0], x[1]);
    } else {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(rowp + 12 * s);
        return unpack_int3_half(p[0], p[1], p[2], h);
    }
}

template <int BITS, int BM, int BN, typename YT>
__global__ __launch_bounds__(256) void qgemm_kernel(const uint8_t *__restrict__ A, const float *__restrict__ sa,
                                                    int n, const uint8_t *__restrict__ W,
                                                    const float *__restrict__ sw, int N, int K,
                                                    YT *__restrict__ y, int64_t ld_y,
                                                    int32_t *__restrict__ acc_out) {
    using F = Fmt<BITS>;
    constexpr int PPR = F::kRowB / 16;             // 16-byte pieces per row per k step
    constexpr int PIECES = (BM + BN) * PPR;
    constexpr int PPT = (PIECES + 255) / 256;      // pieces per thread
    constexpr int TM = BM / 64, TN = BN / 64;      // 32x32 fragments per wave (2 x 2 waves)
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * F::kStride];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int mt = (n + BM - 1) / BM;
    const int bm0 = (blockIdx.x % mt) * BM;
    const int bn0 = (blockIdx.x / mt) * BN;
    const size_t rb = static_cast<size_t>(K) * BITS / 8;  // packed row bytes
    const int nkt = (K + kBK - 1) / kBK;

    v4u stage[PPT];
    auto load_tile = [&](int kt) {
        const int kvalid = min(kBK, K - kt * kBK);          // codes of this step inside the row
        const int bvalid = kvalid * BITS / 8;                // bytes
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + 256 * i;
            v4u val = v4u{0, 0, 0, 0};
            if (p < PIECES) {
                const bool is_a = p < BM * PPR;
                const int q = is_a ? p : p - BM * PPR;
                const int row = q / PPR, part = q % PPR;
                const int grow = (is_a ? bm0 : bn0) + row;
                const bool rvalid = is_a ? grow < n : grow < N;
                const uint8_t *src = (is_a ? A : W) + static_cast<size_t>(grow) * rb + static_cast<size_t>(kt) * F::kRowB + 16 * part;
                if (rvalid) {
                    // int3 rows are only 4-byte aligned when K is not a multiple of 128
                    if (16 * part + 16 <= bvalid && (BITS == 4 || (rb & 15) == 0)) {
                        val = *reinterpret_cast<const v4u *>(src);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (16 * part + 4 * e + 4 <= bvalid) val[e] = reinterpret_cast<const uint32_t *>(src)[e];
                    }
                }
            }
            stage[i] = val;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + 256 * i;
            if (p < PIECES) {
                const int row = p / PPR, part = p % PPR;  // A rows then W rows, contiguous in LDS
                uint32_t *dst = reinterpret_cast<uint32_t *>(&lds[buf][row * F::kStride + 16 * part]);
                if constexpr (F::kStride % 8 == 0) {
                    reinterpret_cast<v2u *>(dst)[0] = v2u{stage[i][0], stage[i][1]};
                    reinterpret_cast<v2u *>(dst)[1] = v2u{stage[i][2], stage[i][3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = stage[i][e];
                }
            }
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) load_tile(kt + 1);
        const uint8_t *la = &lds[buf][0];
        const uint8_t *lw = &lds[buf][BM * F::kStride];
#pragma unroll
        for (int s = 0; s < kBK / 32; ++s) {
            v4i ao[TM], wo[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                ao[i] = lds_operand<BITS>(la + (wm * (BM / 2) + 32 * i + l32) * F::kStride, s, h);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                wo[j] = lds_operand<BITS>(lw + (wn * (BN / 2) + 32 * j + l32) * F::kStride, s, h);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[i], wo[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nkt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds channel l32 of each fragment and tokens 8(v/4) + 4h + v%4
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int ch = bn0 + wn * (BN / 2) + 32 * j + l32;
        const bool cvalid = ch < N;
        const float swj = cvalid ? sw[ch] : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tok = bm0 + wm * (BM / 2) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (cvalid && tok < n) {
                    const int a = acc[i][j][v] >> F::kShift;
                    const float val = (static_cast<float>(a) * sa[tok]) * swj;
                    y[static_cast<int64_t>(tok) * ld_y + ch] = to_out<YT>(val);
                    if (acc_out != nullptr) acc_out[static_cast<int64_t>(tok) * N + ch] = a;
                }
            }
        }
    }
}

template <int BITS, int BM, int BN, typename YT>
hipError_t launch_t(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw, int64_t N,
                    int64_t K, void *y, int64_t ld_y, int32_t *acc_out, hipStream_t s) {
    const int64_t mt = (n + BM - 1) / BM, nt = (N + BN - 1) / BN;
    hipLaunchKernelGGL((qgemm_kernel<BITS, BM, BN, YT>), dim3(static_cast<unsigned>(mt * nt)), dim3(256), 0, s,
                       a, sa, static_cast<int>(n), w, sw, static_cast<int>(N), static_cast<int>(K),
                       static_cast<YT *>(y), ld_y, acc_out);
    return hipGetLastError();
}

template <int BITS, typename YT>
hipError_t launch_b(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw, int64_t N,
                    int64_t K, void *y, int64_t ld_y, int32_t *acc_out, hipStream_t s) {
    if (n <= 64) return launch_t<BITS, 64, 64, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, s);
    return launch_t<BITS, 128, 128, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, s);
}

}  // namespace

hipError_t launch_qgemm(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw,
                        int64_t n_out, int64_t k, int bits, void *y, int y_dtype, int64_t ld_y,
                        int32_t *acc_out, hipStream_t s) {
    if (bits == 4) {
        if (y_dtype == 1) return launch_b<4, uint16_t>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, s);
        return launch_b<4, float>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, s);
    }
    if (y_dtype == 1) return launch_b<3, uint16_t>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, s);
    return launch_b<3, float>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, s);
}

}  // namespace rsq
