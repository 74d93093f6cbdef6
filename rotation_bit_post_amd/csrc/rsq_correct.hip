// Subspace residual rotation (and its fused RMSNorm + per-token quantisation).
//
// Per token row h (ReSpinQuant, zh 2.2 steps 1-3; fr 2C):
//   p = h U            projection onto the r-dimensional subspace
//   c = p M            transform inside it (M = R_sub - I_r)
//   h' = h + c U^T     reprojection added to the residual
// Folding M into the second basis, c U^T = p V^T with V = U M^T, leaves two
// skinny contractions, both on the bf16 matrix cores with float32
// accumulation; the reprojection's accumulator starts at h, so the residual
// add costs nothing. A bfloat16 residual takes bf16 operands (h is exact in
// bf16; U, V and p carry 2^-9 relative rounding, far below the rounding of
// h' itself). A float32 residual also takes the bf16 remainders (hi + lo
// splits, about 2^-17 relative per operand).
//
// Work split: a workgroup owns tb (8 or 16) tokens - the matrix-core N
// dimension is 16, and 8 is used when 16 would leave compute units idle -
// and up to 8 waves (two per SIMD); each wave owns some 32-column chunks of d
// and keeps its slice of the rows in registers from the load until the
// store, so the residual crosses HBM once in and once out. The basis
// operands stream from L2 through a ring of PD chunks per wave. Lane l holds
// token (l % 16) and columns 32c + 8(l / 16) .. +7 of chunk c: the B operand
// of the projection (k-slot e = column 32c + 8g + e) and, by the row order
// chosen for V, also the accumulator layout of the reprojection.
#include <type_traits>

#include <atomic>

#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

namespace {

constexpr int kMaxWaves = kCorrectMaxWaves;

// ------------------------------------------------------------ site layout
// Four parts of d * r_pad bf16 each: U hi, V hi, U lo, V lo (a bf16 residual
// reads only the first two).
// U part: [chunk c][j-block jb (16 wide)][lane][8]: lane l, element e holds
//         U[32c + 8(l/16) + e][16 jb + l%16].
// V part: [chunk c][row-block b][k-block kk (32 wide)][lane][8]: lane l,
//         element e holds V[dd][32 kk + 8(l/16) + e] with
//         dd = 32c + 8((l%16)/4) + 4b + (l%16)%4.
__device__ __forceinline__ size_t u_index(int c, int jb, int lane, int njb) {
    return ((static_cast<size_t>(c) * njb + jb) * 64 + lane) * 8;
}
__device__ __forceinline__ size_t v_index(int c, int b, int kk, int lane, int r32) {
    return (((static_cast<size_t>(c) * 2 + b) * r32 + kk) * 64 + lane) * 8;
}

// One thread per (part, position); position i of a part is its index above.
__global__ void site_prepare_kernel(const float *__restrict__ U, const float *__restrict__ M, int d, int r,
                                    int r_pad, uint16_t *__restrict__ site) {
    const int njb = r_pad / 16, nkk = r_pad / 32;
    const size_t per = static_cast<size_t>(d) * r_pad;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= 2 * per) return;
    const bool is_v = i >= per;
    if (is_v) i -= per;
    const int e = static_cast<int>(i % 8);
    const int lane = static_cast<int>((i / 8) % 64);
    const size_t blk = i / 512;  // U: c * njb + jb ; V: (c * 2 + b) * nkk + kk
    float val;
    if (!is_v) {
        const int jb = static_cast<int>(blk % njb), c = static_cast<int>(blk / njb);
        const int row = 32 * c + 8 * (lane / 16) + e, col = 16 * jb + lane % 16;
        val = col < r ? U[static_cast<size_t>(row) * r + col] : 0.0f;
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
        val = static_cast<float>(v);
    }
    uint16_t hi, lo;
    split_bf16(val, hi, lo);
    const size_t base = is_v ? per : 0;
    site[base + i] = hi;
    site[2 * per + base + i] = lo;
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
    // elements 4b .. 4b+3, rounded to nearest even
    __device__ __forceinline__ void set4(int b, v4f x) {
        raw[2 * b] = pk_bf16(x[0], x[1]);
        raw[2 * b + 1] = pk_bf16(x[2], x[3]);
    }
    // sum of squares of the 8 stored values: bf16 products are exact in
    // float32; float32 adds within the row piece, float64 across pieces
    __device__ __forceinline__ double sumsq() const {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) s = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(raw[q]), as_v2bf(raw[q]), s, false);
        return static_cast<double>(s);
    }
    __device__ __forceinline__ void operands(v8bf &hi, v8bf &lo) const { hi = as_v8bf(raw); (void)lo; }
    __device__ __forceinline__ void shuffle_xor(int mask) {
#pragma unroll
        for (int q = 0; q < 4; ++q) raw[q] = __shfl_xor(raw[q], mask, kWave);
    }
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
    __device__ __forceinline__ void set4(int blk, v4f x) { if (blk == 0) a = x; else b = x; }
    __device__ __forceinline__ double sumsq() const {  // float64 products and adds
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fma(static_cast<double>(get(e)), static_cast<double>(get(e)), s);
        return s;
    }
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
    __device__ __forceinline__ void shuffle_xor(int mask) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            a[q] = __shfl_xor(a[q], mask, kWave);
            b[q] = __shfl_xor(b[q], mask, kWave);
        }
    }
    static constexpr bool kSplit = true;
};

__device__ __forceinline__ v8bf load_op(const uint16_t *p) { return as_v8bf(*reinterpret_cast<const v4u *>(p)); }


// ------------------------------------------------------------ main kernel
// T: uint16_t (bf16) or float. CPW: 32-column chunks per wave. R32: r_pad / 32.
// COLS (small batches, no quantisation): CPW workgroups share a token block;
// each forms the whole projection (U is read through L2 by all of them) but
// reprojects and stores only its slice of nw chunks, one per wave, so a few
// tokens still spread over many compute units. (The quantising call then runs
// the standalone quantiser over the stored rows: measured against one launch
// whose last workgroup per token block quantises the block behind
// device-scope fences, the two launches were as fast at 1 token and faster
// from 8 tokens on, e.g. 10.9 against 14.7 us at 64 tokens.)
// FMT: the code format written when quantising (4, 3 or kFp4), a template
// parameter so that no instance carries the branches of the others.
template <typename T, int CPW, int R32, bool QUANT, bool COLS = false, int FMT = 4>
__global__ __launch_bounds__(64 * kMaxWaves) void correct_kernel(
    const T *__restrict__ h_in, T *__restrict__ h_out, int64_t n, int d, int64_t ld_h,
    const uint16_t *__restrict__ site, int tb, const float *__restrict__ norm_w, float eps,
    uint8_t *__restrict__ codes, float *__restrict__ scales) {
    static_assert(!(COLS && QUANT), "the column-split variant does not quantise");
    constexpr bool SPLIT = Row8<T>::kSplit;
    constexpr int NJB = 2 * R32;               // 16-wide j blocks of the projection
    constexpr int RPS = 32 * R32 + 4;          // LDS row stride of the partial projections (floats)
    // chunks of basis operands in flight per wave: 8 (64 registers) unless
    // the residual slice or the operands are large
    constexpr int HREGS = CPW * 2 * static_cast<int>(sizeof(T));
    constexpr int PD0 = (HREGS >= 128 ? 4 : 8) / (SPLIT ? 2 : 1) / R32;
    constexpr int PD = CPW < PD0 ? CPW : PD0;
    constexpr int NL = SPLIT ? PD : 1;
    __shared__ __attribute__((aligned(16))) float lp[kMaxWaves * 16 * RPS];
    __shared__ double lss[kMaxWaves * 16];
    __shared__ float lam[kMaxWaves * 16];
    __shared__ float lwm[kMaxWaves * 16];

    const int nw = blockDim.x >> 6;
    // the wave index is uniform: keeping it in a scalar register keeps every
    // per-chunk offset below scalar as well
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, tl = lane & 15;
    const int slice = COLS ? static_cast<int>(blockIdx.x % CPW) : 0;
    const int64_t t0 = static_cast<int64_t>(COLS ? blockIdx.x / CPW : blockIdx.x) * tb;
    const int64_t t = t0 + tl;
    const bool valid = tl < tb && t < n;
    // lanes without a token of their own read the block's first row (in
    // bounds, already being fetched) and store nothing
    const int64_t tload = valid ? t : t0;
    const size_t per = static_cast<size_t>(d) * 32 * R32;
    const uint16_t *u_hi = site, *v_hi = site + per, *u_lo = site + 2 * per, *v_lo = site + 3 * per;
    (void)u_lo;
    (void)v_lo;

    // 1. residual slice -> registers; every load in flight at once
    Row8<T> hr[CPW];
#pragma unroll
    for (int m = 0; m < CPW; ++m) hr[m].load(h_in + tload * ld_h + 32 * (w + nw * m) + 8 * g);

    // 2. projection: P^T (r_pad x 16 tokens), partial over this wave's chunks
    v4f acc[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) acc[jb] = v4f{0, 0, 0, 0};
    v8bf uh[PD][NJB], ul[NL][NJB];
#pragma unroll
    for (int p = 0; p < PD; ++p)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            uh[p][jb] = load_op(u_hi + u_index(w + nw * p, jb, lane, NJB));
            if constexpr (SPLIT) ul[p % NL][jb] = load_op(u_lo + u_index(w + nw * p, jb, lane, NJB));
        }
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
        const int sl = m % PD;
        v8bf bh, bl;
        hr[m].operands(bh, bl);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[sl][jb], bh, acc[jb], 0, 0, 0);
            if constexpr (SPLIT) {
                acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul[sl % NL][jb], bh, acc[jb], 0, 0, 0);
                acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[sl][jb], bl, acc[jb], 0, 0, 0);
            }
        }
        if (m + PD < CPW) {
            const int cn = w + nw * (m + PD);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                uh[sl][jb] = load_op(u_hi + u_index(cn, jb, lane, NJB));
                if constexpr (SPLIT) ul[sl % NL][jb] = load_op(u_lo + u_index(cn, jb, lane, NJB));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // first reprojection operands, in flight during the reduction below
    v8bf vh[PD][2][R32], vl[NL][2][R32];
#pragma unroll
    for (int p = 0; p < (COLS ? 0 : PD); ++p)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int kk = 0; kk < R32; ++kk) {
                vh[p][b][kk] = load_op(v_hi + v_index(w + nw * p, b, kk, lane, R32));
                if constexpr (SPLIT) vl[p % NL][b][kk] = load_op(v_lo + v_index(w + nw * p, b, kk, lane, R32));
            }

    // 3. sum the waves' partial projections (the same order in every wave)
    //    and take P^T as the reprojection's B operand (k-slot e = column 8g + e)
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
        *reinterpret_cast<v4f *>(&lp[(w * 16 + tl) * RPS + 16 * jb + 4 * g]) = acc[jb];
    __syncthreads();
    v8bf ph[R32], pl[R32];
#pragma unroll
    for (int kk = 0; kk < R32; ++kk) {
        v4f p0 = v4f{0, 0, 0, 0}, p1 = p0;
        for (int ww = 0; ww < nw; ++ww) {
            const float *src = &lp[(ww * 16 + tl) * RPS + 32 * kk + 8 * g];
            p0 += *reinterpret_cast<const v4f *>(src);
            p1 += *reinterpret_cast<const v4f *>(src + 4);
        }
        v4u hi{pk_bf16(p0[0], p0[1]), pk_bf16(p0[2], p0[3]), pk_bf16(p1[0], p1[1]), pk_bf16(p1[2], p1[3])};
        ph[kk] = as_v8bf(hi);
        if constexpr (SPLIT) {
            const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            v4u lo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float h0 = __uint_as_float(hi[q] << 16), h1 = __uint_as_float(hi[q] & 0xFFFF0000u);
                lo[q] = pk_bf16(pv[2 * q] - h0, pv[2 * q + 1] - h1);
            }
            pl[kk] = as_v8bf(lo);
        }
    }

    if constexpr (COLS) {
        // 4'. this workgroup's slice: chunk slice * nw + w for wave w, its
        //     residual read again (an L2 hit: the projection just read it)
        const int c = slice * nw + w;
        Row8<T> hc;
        hc.load(h_in + tload * ld_h + 32 * c + 8 * g);
        v8bf vc[2][R32], vcl[2][R32];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int kk = 0; kk < R32; ++kk) {
                vc[b][kk] = load_op(v_hi + v_index(c, b, kk, lane, R32));
                if constexpr (SPLIT) vcl[b][kk] = load_op(v_lo + v_index(c, b, kk, lane, R32));
            }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            v4f cacc;
#pragma unroll
            for (int v = 0; v < 4; ++v) cacc[v] = hc.get(4 * b + v);
#pragma unroll
            for (int kk = 0; kk < R32; ++kk) {
                cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vc[b][kk], ph[kk], cacc, 0, 0, 0);
                if constexpr (SPLIT) {
                    cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcl[b][kk], ph[kk], cacc, 0, 0, 0);
                    cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vc[b][kk], pl[kk], cacc, 0, 0, 0);
                }
            }
            hc.set4(b, cacc);
        }
        if (valid) hc.store(h_out + t * ld_h + 32 * c + 8 * g);
        return;
    }

    // 4. reprojection + residual (C: 16 columns of d x 16 tokens, seeded with
    //    h), rounded to the storage type
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
        const int sl = m % PD;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            v4f cacc;
#pragma unroll
            for (int v = 0; v < 4; ++v) cacc[v] = hr[m].get(4 * b + v);
#pragma unroll
            for (int kk = 0; kk < R32; ++kk) {
                cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[sl][b][kk], ph[kk], cacc, 0, 0, 0);
                if constexpr (SPLIT) {
                    cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl[sl % NL][b][kk], ph[kk], cacc, 0, 0, 0);
                    cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[sl][b][kk], pl[kk], cacc, 0, 0, 0);
                }
            }
            hr[m].set4(b, cacc);
        }
        if (m + PD < CPW) {
            const int cn = w + nw * (m + PD);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int kk = 0; kk < R32; ++kk) {
                    vh[sl][b][kk] = load_op(v_hi + v_index(cn, b, kk, lane, R32));
                    if constexpr (SPLIT) vl[sl % NL][b][kk] = load_op(v_lo + v_index(cn, b, kk, lane, R32));
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int m = 0; m < CPW; ++m) hr[m].opaque();
    // Statistics, scale, quantisation and packing of NC chunks per lane: chunk
    // m of this lane is global chunk w + nw * (m + base) of token t0 + tok.
    // PAIR: lanes l and l ^ 8 hold two halves of one token's chunks.
    auto quant_epilogue = [&](auto nc_c, auto pair_c, int base, int tok) {
        constexpr int NC = decltype(nc_c)::value;
        constexpr bool PAIR = decltype(pair_c)::value;
        const int64_t tt = t0 + tok;
        const bool ok = tok < tb && tt < n;
        double ss = 0.0;
        float am = 0.0f;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            ss += hr[m].sumsq();
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(hr[m].get(e)));
        }
        if constexpr (PAIR) {
            ss += shfl_xor_f64(ss, 8);
            am = wave_max_xor(am, 8);
        }
        ss += shfl_xor_f64(ss, 16);
        ss += shfl_xor_f64(ss, 32);
        am = wave_max_xor(am, 16);
        am = wave_max_xor(am, 32);
        if (g == 0 && (!PAIR || tl < 8)) {
            lss[w * 16 + tok] = ss;
            lam[w * 16 + tok] = am;
        }
        __syncthreads();
        double tot = 0.0;
        float amax = 0.0f;
        for (int ww = 0; ww < nw; ++ww) {
            tot += lss[ww * 16 + tok];
            amax = fmaxf(amax, lam[ww * 16 + tok]);
        }
        const float inv = static_cast<float>(1.0 / sqrt(tot / static_cast<double>(d) + static_cast<double>(eps)));
        float mval;
        if (norm_w == nullptr) {
            mval = amax * inv;  // rounding is monotone: max|x * inv| = max|x| * inv
        } else {
            float a2 = 0.0f;
#pragma unroll
            for (int m = 0; m < NC; ++m) {
                const float *wp = norm_w + 32 * (w + nw * (m + base)) + 8 * g;
                const v4f w0 = *reinterpret_cast<const v4f *>(wp), w1 = *reinterpret_cast<const v4f *>(wp + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) a2 = fmaxf(a2, fabsf((hr[m].get(e) * inv) * (e < 4 ? w0[e] : w1[e - 4])));
            }
            if constexpr (PAIR) a2 = wave_max_xor(a2, 8);
            a2 = wave_max_xor(a2, 16);
            a2 = wave_max_xor(a2, 32);
            if (g == 0 && (!PAIR || tl < 8)) lwm[w * 16 + tok] = a2;
            __syncthreads();
            mval = 0.0f;
            for (int ww = 0; ww < nw; ++ww) mval = fmaxf(mval, lwm[ww * 16 + tok]);
        }
#pragma unroll
        for (int m = 0; m < NC; ++m) hr[m].opaque();
        const float *nw_q = norm_w;
        asm volatile("" : "+s"(nw_q));  // reload the weights below instead of keeping them live
        constexpr int qmax = FMT == 4 ? 7 : 3;
        const float s = __fdiv_rn(mval, static_cast<float>(qmax));
        const float inv_s = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
        const size_t rowb = FMT == 3 ? static_cast<size_t>(d) * 3 / 8 : static_cast<size_t>(d) / 2;
        auto quant_chunk = [&](int m, const float *wts) {
            const int c = w + nw * (m + base);
            uint32_t u[8];
            if (wts != nullptr) {
                const v4f w0 = *reinterpret_cast<const v4f *>(wts + 32 * c + 8 * g);
                const v4f w1 = *reinterpret_cast<const v4f *>(wts + 32 * c + 8 * g + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] = quant_bits((hr[m].get(e) * inv) * (e < 4 ? w0[e] : w1[e - 4]), s, inv_s);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] = quant_bits(hr[m].get(e) * inv, s, inv_s);
            }
            if constexpr (FMT == 4) {
                uint32_t word = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) word |= (u[e] & 0xFu) << (4 * e);
                if (ok) *reinterpret_cast<uint32_t *>(codes + tt * rowb + 16 * c + 4 * g) = word;
            } else if constexpr (FMT == kFp4) {   // word g of the chunk's 32-code group
                if (ok) *reinterpret_cast<uint32_t *>(codes + tt * rowb + 16 * c + 4 * g) = fp4_word(u);
            } else {
                uint32_t own, low[3];
                int3_lane_parts(u, own, low);
                const int src = 48 + tl;  // the g = 3 lane of this token and chunk
                const uint32_t l0 = __shfl(low[0], src, kWave), l1 = __shfl(low[1], src, kWave),
                               l2 = __shfl(low[2], src, kWave);
                const uint32_t word = own | (g == 0 ? l0 : (g == 1 ? l1 : l2));
                if (ok && g < 3) *reinterpret_cast<uint32_t *>(codes + tt * rowb + 12 * c + 4 * g) = word;
            }
            if (ok) hr[m].store(h_out + tt * ld_h + 32 * c + 8 * g);
        };
        if (nw_q != nullptr) {
#pragma unroll
            for (int m = 0; m < NC; ++m) {
                quant_chunk(m, nw_q);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int m = 0; m < NC; ++m) {
                quant_chunk(m, nullptr);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (ok && w == 0 && g == 0 && base == 0) scales[tt] = s;
    };

    if constexpr (QUANT) {
        // 5-6. RMSNorm statistics, scale, quantisation and packing. With 8-token
        // blocks the lanes of tokens 8-15 hold no token of their own: they take
        // over the upper half of the chunks of token (l % 16) - 8, which halves
        // the per-element work of every lane.
        if constexpr (CPW >= 2 && CPW <= 16) {   // (32 chunks: registers are too tight for two variants)
            if (tb <= 8) {
#pragma unroll
                for (int m = 0; m < CPW / 2; ++m) {
                    Row8<T> up = hr[m + CPW / 2];
                    up.shuffle_xor(8);
                    if (tl >= 8) hr[m] = up;
                }
                quant_epilogue(std::integral_constant<int, CPW / 2>{}, std::true_type{}, tl >= 8 ? CPW / 2 : 0, tl & 7);
            } else {
                quant_epilogue(std::integral_constant<int, CPW>{}, std::false_type{}, 0, tl);
            }
        } else {
            quant_epilogue(std::integral_constant<int, CPW>{}, std::false_type{}, 0, tl);
        }
    }

    // 7. h' -> HBM (the quantising variant stores it in its epilogue)
    if constexpr (!QUANT) {
        if (valid) {
#pragma unroll
            for (int m = 0; m < CPW; ++m) hr[m].store(h_out + t * ld_h + 32 * (w + nw * m) + 8 * g);
        }
    }
}

// Token block size and whether the column-split form is taken (few tokens:
// CPW workgroups per token block; not in place, since other workgroups of the
// block still read the residual).
struct CorrectPlan {
    int tb;
    int64_t blocks;
    bool cols;
};
CorrectPlan correct_plan(int64_t n, int cpw, bool in_place, int cus) {
    CorrectPlan p;
    p.tb = (n + 15) / 16 >= cus ? 16 : 8;
    p.blocks = (n + p.tb - 1) / p.tb;
    p.cols = cpw >= 4 && !in_place && p.blocks * cpw <= cus;
    return p;
}

template <typename T, int CPW, int R32, bool QUANT>
hipError_t launch_t(const void *h_in, void *h_out, int64_t n, int d, int64_t ld_h, const void *site, int nw,
                    const float *norm_w, float eps, int bits, uint8_t *codes, float *scales, hipStream_t s) {
    const CorrectPlan plan = correct_plan(n, CPW, h_in == h_out, device_cus());
    const int tb = plan.tb;
    const int64_t blocks = plan.blocks;
    const T *hi = static_cast<const T *>(h_in);
    T *ho = static_cast<T *>(h_out);
    const uint16_t *st = static_cast<const uint16_t *>(site);
    // few tokens: the column-split correction; the quantising call then
    // normalises and quantises the stored rows with the standalone quantiser
    if constexpr (CPW >= 4) {
        if (plan.cols) {
            if (!grid_fits(blocks * CPW, 64 * nw)) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((correct_kernel<T, CPW, R32, false, true>), dim3(static_cast<unsigned>(blocks * CPW)),
                               dim3(64 * nw), 0, s, hi, ho, n, d, ld_h, st, tb, nullptr, 0.0f, nullptr, nullptr);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || !QUANT) return e;
            return launch_quant(h_out, sizeof(T) == 2 ? 1 : 0, n, d, ld_h, true, norm_w, eps, bits, codes, scales, s);
        }
    }
    if (!grid_fits(blocks, 64 * nw)) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * nw);
    if constexpr (!QUANT) {
        hipLaunchKernelGGL((correct_kernel<T, CPW, R32, false>), grid, block, 0, s, hi, ho, n, d, ld_h, st, tb, norm_w,
                           eps, codes, scales);
    } else if (bits == 4) {
        hipLaunchKernelGGL((correct_kernel<T, CPW, R32, true, false, 4>), grid, block, 0, s, hi, ho, n, d, ld_h, st, tb,
                           norm_w, eps, codes, scales);
    } else if (bits == kFp4) {
        hipLaunchKernelGGL((correct_kernel<T, CPW, R32, true, false, kFp4>), grid, block, 0, s, hi, ho, n, d, ld_h, st,
                           tb, norm_w, eps, codes, scales);
    } else {
        hipLaunchKernelGGL((correct_kernel<T, CPW, R32, true, false, 3>), grid, block, 0, s, hi, ho, n, d, ld_h, st, tb,
                           norm_w, eps, codes, scales);
    }
    return hipGetLastError();
}

template <typename T, int CPW, bool QUANT>
hipError_t launch_r(int r32, const void *h_in, void *h_out, int64_t n, int d, int64_t ld_h, const void *site,
                    int nw, const float *norm_w, float eps, int bits, uint8_t *codes, float *scales, hipStream_t s) {
    if (r32 == 1)
        return launch_t<T, CPW, 1, QUANT>(h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
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
        default:
            if constexpr (sizeof(T) == 2)
                return launch_r<T, 32, QUANT>(r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales,
                                              s);
            return hipErrorInvalidValue;
    }
}

}  // namespace

int device_cus() {
    // per-device cache; callers on several threads may fill it concurrently
    // (they store the same value)
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
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
                          uint8_t *codes, float *scales, void *ws, hipStream_t s) {
    (void)ws;   // see correct_workspace_bytes
    int nw = 0, cpw = 0;
    if (!correct_geometry(d, h_dtype == 0, &nw, &cpw)) return hipErrorInvalidValue;
    const int r32 = rank_pad(r) / 32;
    if (h_dtype == 1) {
        if (quant)
            return launch_c<uint16_t, true>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes,
                                            scales, s);
        return launch_c<uint16_t, false>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales,
                                         s);
    }
    if (quant)
        return launch_c<float, true>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
    return launch_c<float, false>(cpw, r32, h_in, h_out, n, d, ld_h, site, nw, norm_w, eps, bits, codes, scales, s);
}

size_t correct_workspace_bytes(int64_t n, int64_t d) {
    // no correction kernel needs scratch: every exchange stays inside a
    // workgroup (LDS), and the small-batch site runs as two launches rather
    // than one whose workgroups meet through device memory (see correct_kernel)
    (void)n; (void)d;
    return 0;
}

}  // namespace rsq
