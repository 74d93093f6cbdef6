// Subspace residual rotation (and its fused RMSNorm + per-token quantisation).
//
// Per token row h (ReSpinQuant, zh 2.2 steps 1-3; fr 2C):
//   p = h U            projection onto the r-dimensional subspace
//   c = p M            transform inside it (M = R_sub - I_r)
//   h' = h + c U^T     reprojection added to the residual
// Folding M into the second basis, c U^T = p V^T with V = U M^T, leaves two
// skinny contractions. Both run on the bf16 matrix cores with a hi/lo split
// of the float32 operands (about 2^-17 relative each) and float32
// accumulation; the reprojection's accumulator starts at h, so the residual
// add costs nothing.
//
// Work split: a workgroup owns 16 tokens (the matrix-core N dimension) and
// up to 8 waves (two per SIMD, 256 registers each); each wave owns some 32-column chunks of d and keeps its
// slice of the 16 rows in registers from the load until the store, so the
// residual crosses HBM once in and once out. Lane l holds token (l % 16) and
// columns 32c + 8(l / 16) .. +7 of chunk c: the B operand of the projection
// (k-slot e = column 32c + 8g + e) and, by the row order chosen for V, also
// the accumulator layout of the reprojection.
#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

namespace {

constexpr int kTok = 16;        // tokens per workgroup
constexpr int kMaxWaves = 8;

// ------------------------------------------------------------ site layout
// U part: [chunk c][j-block jb (16 wide)][hi|lo][lane][8]: lane l, element e
//         holds U[32c + 8(l/16) + e][16 jb + l%16].
// V part: [chunk c][row-block b][k-block kk (32 wide)][hi|lo][lane][8]: lane l,
//         element e holds V[d][32 kk + 8(l/16) + e] with
//         d = 32c + 8((l%16)/4) + 4b + (l%16)%4.
__device__ __forceinline__ size_t u_index(int c, int jb, int hl, int lane, int njb) {
    return ((static_cast<size_t>(c) * njb + jb) * 2 + hl) * 512 + lane * 8;
}
__device__ __forceinline__ size_t v_index(int c, int b, int kk, int hl, int lane, int nkk) {
    return (((static_cast<size_t>(c) * 2 + b) * nkk + kk) * 2 + hl) * 512 + lane * 8;
}

__global__ void site_prepare_kernel(const float *__restrict__ U, const float *__restrict__ M, int d, int r,
                                    int r_pad, uint16_t *__restrict__ site) {
    const int njb = r_pad / 16, nkk = r_pad / 32;
    const size_t half = static_cast<size_t>(d) * r_pad * 2;  // elements of the U part (hi + lo)
    const size_t per = static_cast<size_t>(d) * r_pad;       // (chunk, block, lane, e) positions
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= 2 * per) return;
    const bool is_v = i >= per;
    if (is_v) i -= per;
    const int e = static_cast<int>(i % 8);
    const int lane = static_cast<int>((i / 8) % 64);
    const size_t blk = i / 512;  // U: c * njb + jb ; V: (c * 2 + b) * nkk + kk
    if (!is_v) {
        const int jb = static_cast<int>(blk % njb), c = static_cast<int>(blk / njb);
        const int row = 32 * c + 8 * (lane / 16) + e, col = 16 * jb + lane % 16;
        const float u = col < r ? U[static_cast<size_t>(row) * r + col] : 0.0f;
        uint16_t hi, lo;
        split_bf16(u, hi, lo);
        site[u_index(c, jb, 0, lane, njb) + e] = hi;
        site[u_index(c, jb, 1, lane, njb) + e] = lo;
    } else {
        const int kk = static_cast<int>(blk % nkk);
        const int b = static_cast<int>((blk / nkk) % 2), c = static_cast<int>(blk / nkk / 2);
        const int i16 = lane % 16;
        const int row = 32 * c + 8 * (i16 / 4) + 4 * b + i16 % 4;
        const int col = 32 * kk + 8 * (lane / 16) + e;
        double v = 0.0;
        if (col < r)
            for (int m = 0; m < r; ++m)
                v += static_cast<double>(U[static_cast<size_t>(row) * r + m]) * static_cast<double>(M[static_cast<size_t>(col) * r + m]);
        const uint16_t hi = f32_to_bf16(static_cast<float>(v));
        const uint16_t lo = f32_to_bf16(static_cast<float>(v - static_cast<double>(bf16_to_f32(hi))));
        site[half + v_index(c, b, kk, 0, lane, nkk) + e] = hi;
        site[half + v_index(c, b, kk, 1, lane, nkk) + e] = lo;
    }
}

// ------------------------------------------------------ residual storage
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {  // bfloat16: 8 values in 16 bytes
    v4u raw;
    __device__ __forceinline__ void load(const uint16_t *p) { raw = *reinterpret_cast<const v4u *>(p); }
    __device__ __forceinline__ void store(uint16_t *p) const { *reinterpret_cast<v4u *>(p) = raw; }
    __device__ __forceinline__ void zero() { raw = v4u{0, 0, 0, 0}; }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = raw[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    __device__ __forceinline__ void set(int e, float f) {  // rounds to nearest even
        const uint32_t b = f32_to_bf16(f);
        uint32_t w = raw[e >> 1];
        w = (e & 1) ? ((w & 0xFFFFu) | (b << 16)) : ((w & 0xFFFF0000u) | b);
        raw[e >> 1] = w;
    }
    __device__ __forceinline__ void operands(v8bf &hi, v8bf &lo) const { hi = as_v8bf(raw); (void)lo; }
    // Hide the value from common-subexpression elimination, so unpacked copies
    // are recomputed per phase instead of being kept live across phases.
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(raw)); }
    static constexpr bool kSplit = false;
};
template <> struct Row8<float> {  // float32: 8 values in 32 bytes
    v4f a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const v4f *>(p);
        b = *reinterpret_cast<const v4f *>(p + 4);
    }
    __device__ __forceinline__ void store(float *p) const {
        *reinterpret_cast<v4f *>(p) = a;
        *reinterpret_cast<v4f *>(p + 4) = b;
    }
    __device__ __forceinline__ void zero() { a = v4f{0, 0, 0, 0}; b = a; }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
    __device__ __forceinline__ void set(int e, float f) { if (e < 4) a[e] = f; else b[e - 4] = f; }
    __device__ __forceinline__ void operands(v8bf &hi, v8bf &lo) const {
        v4u h, l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint16_t h0, l0, h1, l1;
            split_bf16(get(2 * q), h0, l0);
            split_bf16(get(2 * q + 1), h1, l1);
            h[q] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
            l[q] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
        }
        hi = as_v8bf(h);
        lo = as_v8bf(l);
    }
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(a), "+v"(b)); }
    static constexpr bool kSplit = true;
};

__device__ __forceinline__ v8bf load_op(const uint16_t *p) { return as_v8bf(*reinterpret_cast<const v4u *>(p)); }

// ------------------------------------------------------------ main kernel
// T: uint16_t (bf16) or float. CPW: 32-column chunks per wave. R32: r_pad / 32.
template <typename T, int CPW, int R32, bool QUANT>
__global__ __launch_bounds__(512) void correct_kernel(
    const T *__restrict__ h_in, T *__restrict__ h_out, int64_t n, int d, int64_t ld_h,
    const uint16_t *__restrict__ site, int nw, const float *__restrict__ norm_w, float eps, int bits,
    uint8_t *__restrict__ codes, float *__restrict__ scales) {
    constexpr int NJB = 2 * R32;  // 16-wide j blocks
    __shared__ float red[kMaxWaves][kTok][33];
    __shared__ __attribute__((aligned(16))) uint16_t pbuf[2][kTok][R32 * 32 + 8];
    __shared__ double ssq[kMaxWaves][kTok];
    __shared__ float amx[kMaxWaves][kTok];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, tl = lane & 15;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTok + tl;
    const bool valid = t < n;
    const size_t vbase = static_cast<size_t>(d) * R32 * 32 * 2;  // start of the V part

    // 1. residual slice -> registers
    Row8<T> hr[CPW];
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
        const int c = w + nw * m;
        if (valid) hr[m].load(h_in + t * ld_h + 32 * c + 8 * g);
        else hr[m].zero();
    }

    // 2. projection: P^T (r_pad x 16 tokens) partial over this wave's chunks.
    //    Operands of chunk m + 1 are loaded while chunk m is multiplied.
    v4f acc[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) acc[jb] = v4f{0, 0, 0, 0};
    v8bf uh[2][NJB], ul[2][NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
        uh[0][jb] = load_op(site + u_index(w, jb, 0, lane, NJB));
        ul[0][jb] = load_op(site + u_index(w, jb, 1, lane, NJB));
    }
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
        const int cur = m & 1;
        if (m + 1 < CPW) {
            const int cn = w + nw * (m + 1);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                uh[cur ^ 1][jb] = load_op(site + u_index(cn, jb, 0, lane, NJB));
                ul[cur ^ 1][jb] = load_op(site + u_index(cn, jb, 1, lane, NJB));
            }
        }
        v8bf bh, bl;
        hr[m].operands(bh, bl);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[cur][jb], bh, acc[jb], 0, 0, 0);
            acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul[cur][jb], bh, acc[jb], 0, 0, 0);
            if constexpr (Row8<T>::kSplit)
                acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[cur][jb], bl, acc[jb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // one chunk of operands in flight at a time
    }

    // first reprojection operands, loaded before the reduction so their
    // latency overlaps it (steps are (chunk m, row block b), 2 per chunk)
    v8bf vh[2][R32], vl[2][R32];
#pragma unroll
    for (int kk = 0; kk < R32; ++kk) {
        vh[0][kk] = load_op(site + vbase + v_index(w, 0, kk, 0, lane, R32));
        vl[0][kk] = load_op(site + vbase + v_index(w, 0, kk, 1, lane, R32));
    }

    // 3. sum the partial projections over waves, 32 columns of P at a time,
    //    and keep P as bf16 hi + lo in LDS
#pragma unroll
    for (int kk = 0; kk < R32; ++kk) {
#pragma unroll
        for (int jh = 0; jh < 2; ++jh)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[w][tl][16 * jh + 4 * g + v] = acc[2 * kk + jh][v];
        __syncthreads();
        for (int idx = threadIdx.x; idx < kTok * 32; idx += blockDim.x) {
            const int tok = idx >> 5, j = idx & 31;
            float s = 0.0f;
            for (int ww = 0; ww < nw; ++ww) s += red[ww][tok][j];
            uint16_t hi, lo;
            split_bf16(s, hi, lo);
            pbuf[0][tok][32 * kk + j] = hi;
            pbuf[1][tok][32 * kk + j] = lo;
        }
        __syncthreads();
    }

    // 4. reprojection + residual: C (16 rows of d x 16 tokens) starts at h
    v8bf ph[R32], pl[R32];
#pragma unroll
    for (int kk = 0; kk < R32; ++kk) {
        ph[kk] = load_op(&pbuf[0][tl][32 * kk + 8 * g]);
        pl[kk] = load_op(&pbuf[1][tl][32 * kk + 8 * g]);
    }
#pragma unroll
    for (int st = 0; st < 2 * CPW; ++st) {
        const int m = st >> 1, b = st & 1, cur = st & 1;
        if (st + 1 < 2 * CPW) {
            const int cn = w + nw * ((st + 1) >> 1), bn = (st + 1) & 1;
#pragma unroll
            for (int kk = 0; kk < R32; ++kk) {
                vh[cur ^ 1][kk] = load_op(site + vbase + v_index(cn, bn, kk, 0, lane, R32));
                vl[cur ^ 1][kk] = load_op(site + vbase + v_index(cn, bn, kk, 1, lane, R32));
            }
        }
        v4f cacc;
#pragma unroll
        for (int v = 0; v < 4; ++v) cacc[v] = hr[m].get(4 * b + v);
#pragma unroll
        for (int kk = 0; kk < R32; ++kk) {
            cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[cur][kk], ph[kk], cacc, 0, 0, 0);
            cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl[cur][kk], ph[kk], cacc, 0, 0, 0);
            cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[cur][kk], pl[kk], cacc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) hr[m].set(4 * b + v, cacc[v]);
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int m = 0; m < CPW; ++m) hr[m].opaque();
    if constexpr (QUANT) {
        // 5. RMSNorm statistics of the stored (rounded) h'
        double ss = 0.0;
        float am = 0.0f;
#pragma unroll
        for (int m = 0; m < CPW; ++m) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = hr[m].get(e);
                ss = fma(static_cast<double>(x), static_cast<double>(x), ss);
                am = fmaxf(am, fabsf(x));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        ss += shfl_xor_f64(ss, 16);
        ss += shfl_xor_f64(ss, 32);
        am = wave_max_xor(am, 16);
        am = wave_max_xor(am, 32);
        if (g == 0) { ssq[w][tl] = ss; amx[w][tl] = am; }
        __syncthreads();
        double tot = 0.0;
        float amax = 0.0f;
        for (int ww = 0; ww < nw; ++ww) { tot += ssq[ww][tl]; amax = fmaxf(amax, amx[ww][tl]); }
        const float inv = static_cast<float>(1.0 / sqrt(tot / static_cast<double>(d) + static_cast<double>(eps)));
        float mval;
        if (norm_w == nullptr) {
            mval = amax * inv;  // rounding is monotone: max|x * inv| = max|x| * inv
        } else {
            float a2 = 0.0f;
#pragma unroll
            for (int m = 0; m < CPW; ++m) {
                const int c = w + nw * m;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    a2 = fmaxf(a2, fabsf((hr[m].get(e) * inv) * norm_w[32 * c + 8 * g + e]));
            }
            a2 = wave_max_xor(a2, 16);
            a2 = wave_max_xor(a2, 32);
            __syncthreads();
            if (g == 0) amx[w][tl] = a2;
            __syncthreads();
            mval = 0.0f;
            for (int ww = 0; ww < nw; ++ww) mval = fmaxf(mval, amx[ww][tl]);
        }
#pragma unroll
        for (int m = 0; m < CPW; ++m) hr[m].opaque();
        const float *nw_q = norm_w;
        asm volatile("" : "+s"(nw_q));  // reload the weights below instead of keeping them live
        const int qmax = (1 << (bits - 1)) - 1;
        const float s = __fdiv_rn(mval, static_cast<float>(qmax));
        const float inv_s = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
        const size_t rowb = bits == 4 ? static_cast<size_t>(d) / 2 : static_cast<size_t>(d) * 3 / 8;

        // 6. quantise + pack
#pragma unroll
        for (int m = 0; m < CPW; ++m) {
            const int c = w + nw * m;
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = hr[m].get(e) * inv;
                if (nw_q != nullptr) a *= nw_q[32 * c + 8 * g + e];
                q[e] = s > 0.0f ? quant_code(a, s, inv_s, qmax) : 0;
            }
            if (bits == 4) {
                if (valid)
                    *reinterpret_cast<uint32_t *>(codes + t * rowb + 16 * c + 4 * g) = pack_int4x8(q);
            } else {
                uint32_t w0, w1, w2;
                int3_part(q, g, w0, w1, w2);
                w0 |= __shfl_xor(w0, 16, kWave); w0 |= __shfl_xor(w0, 32, kWave);
                w1 |= __shfl_xor(w1, 16, kWave); w1 |= __shfl_xor(w1, 32, kWave);
                w2 |= __shfl_xor(w2, 16, kWave); w2 |= __shfl_xor(w2, 32, kWave);
                if (valid && g < 3)
                    *reinterpret_cast<uint32_t *>(codes + t * rowb + 12 * c + 4 * g) = g == 0 ? w0 : (g == 1 ? w1 : w2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (valid && w == 0 && g == 0) scales[t] = s;
    }

    // 7. h' -> HBM
    if (valid) {
#pragma unroll
        for (int m = 0; m < CPW; ++m) hr[m].store(h_out + t * ld_h + 32 * (w + nw * m) + 8 * g);
    }
}

template <typename T, int CPW, int R32, bool QUANT>
hipError_t launch_t(const void *h_in, void *h_out, int64_t n, int d, int64_t ld_h, const void *site, int nw,
                    const float *norm_w, float eps, int bits, uint8_t *codes, float *scales, hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>((n + kTok - 1) / kTok);
    hipLaunchKernelGGL((correct_kernel<T, CPW, R32, QUANT>), dim3(blocks), dim3(64 * nw), 0, s,
                       static_cast<const T *>(h_in), static_cast<T *>(h_out), n, d, ld_h,
                       static_cast<const uint16_t *>(site), nw, norm_w, eps, bits, codes, scales);
    return hipGetLastError();
}

template <typename T, int CPW, bool QUANT>
hipError_t launch_r(int r32, const void *h_in, void *h_out, int64_t n, int d, int64_t ld_h, const void *site,
                    int nw, const float *norm_w, float eps, int bits, uint8_t *codes, float *scales, hipStream_t s) {
    if (r32 == 1) return launch_t<T, CPW, 1, QUANT>(h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
    return launch_t<T, CPW, 2, QUANT>(h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
}

template <typename T, bool QUANT>
hipError_t launch_c(int cpw, int r32, const void *h_in, void *h_out, int64_t n, int d, int64_t ld_h,
                    const void *site, int nw, const float *norm_w, float eps, int bits, uint8_t *codes,
                    float *scales, hipStream_t s) {
    switch (cpw) {
        case 1: return launch_r<T, 1, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
        case 2: return launch_r<T, 2, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
        case 4: return launch_r<T, 4, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
        case 8: return launch_r<T, 8, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
        case 16: return launch_r<T, 16, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
        default: return launch_r<T, 32, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
    }
}

}  // namespace

bool correct_geometry(int64_t d, int *waves, int *chunks_per_wave) {
    if (d <= 0 || d % 32) return false;
    const int64_t nch = d / 32;
    for (int cpw : {1, 2, 4, 8, 16, 32}) {
        if (nch % cpw == 0 && nch / cpw <= kMaxWaves) {
            *waves = static_cast<int>(nch / cpw);
            *chunks_per_wave = cpw;
            return true;
        }
    }
    return false;
}

hipError_t launch_site_prepare(const float *U, const float *M, int d, int r, void *site, hipStream_t s) {
    const int r_pad = rank_pad(r);
    const size_t total = static_cast<size_t>(2) * d * r_pad;
    const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
    hipLaunchKernelGGL(site_prepare_kernel, dim3(blocks), dim3(256), 0, s, U, M, d, r, r_pad,
                       static_cast<uint16_t *>(site));
    return hipGetLastError();
}

hipError_t launch_correct(const void *h_in, void *h_out, int h_dtype, int64_t n, int d, int64_t ld_h,
                          const void *site, int r, bool quant, const float *norm_w, float eps, int bits,
                          uint8_t *codes, float *scales, hipStream_t s) {
    int nw = 0, cpw = 0;
    if (!correct_geometry(d, &nw, &cpw)) return hipErrorInvalidValue;
    const int r32 = rank_pad(r) / 32;
    if (h_dtype == 1) {
        if (quant) return launch_c<uint16_t, true>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
        return launch_c<uint16_t, false>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
    }
    if (quant) return launch_c<float, true>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
    return launch_c<float, false>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
}

}  // namespace rsq
