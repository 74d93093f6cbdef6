// Quantised linear: int4 / int3 codes on the int8 matrix cores.
//
//   acc[t, j] = sum_k a[t, k] w[j, k]            (int32, exact)
//   y[t, j]   = (float(acc) * s_a[t]) * s_w[j]
//
// Packed tiles are loaded from HBM/L2, widened to int8 once per workgroup on
// their way into LDS (double buffered, one barrier per 128-code k step, placed
// so that the multiplies of the step's last 32 codes run across it) and read
// back with 16-byte LDS loads straight into v_mfma_i32_32x32x32_i8.
// Widening only moves each code's bits to the top of its byte, so the matrix
// core multiplies 16*a by 16*w (int4) or 32*a by 32*w (int3); the epilogue
// shifts the exact accumulator back. Every widened code lies in [-128, 112],
// so a product is at most 2^14 in magnitude and with K <= 65536 (checked at
// the boundary) the scaled sum stays below 2^30. The k order inside a 32-code
// step is permuted the same way for both operands, which leaves the dot
// products unchanged.
//
// On the 256 x 128 tiles and the decode-size 32 x 32 and 64 x 64 tiles, int4
// codes instead go into LDS packed, as loaded, in 256-code k steps: each
// 16-byte LDS read is one 32-code group, widened in registers, whose low and
// high 8 bytes feed two multiplies (the same split for both operands). Per
// code that halves the LDS writes, the LDS reads and the barriers (and the
// k steps of a tile), at the cost of widening per wave instead of once per
// workgroup; these tiles have the registers for it (measured on MI355X:
// 2048 tokens, o 37.0 against 38.8 us, down 85.0 against 97.4 us; 64 tokens,
// q|k|v 11.4 against 13.6 us). The 256 x 192 and 256 x 256 tiles gain
// nothing from it and keep the widened form.
//
// Matrix-core roles: A = activations (rows = tokens), B = weights (columns =
// output channels). The epilogue stages the bf16 tile in LDS and writes it
// with 16-byte row-contiguous stores.
//
// 3-bit codes held as fp4 (rsq_qgemm_fp4) take the MX matrix cores: a code c
// in [-3, 3] is exact in fp4 e2m1 as c / 2 (sign and magnitude, 0.5 steps), so
// with a block scale of 2 on both operands v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies the codes themselves. Every product is an integer of magnitude
// at most 9 and every partial sum at most 9 K <= 589824 < 2^24, so the
// float32 accumulation is exact in any order and converts back to the same
// int32 sums. The fp4 multiply takes 64 codes per instruction at the rate the
// int8 one takes 32; the fp4 tiles go into LDS as loaded (half the LDS bytes
// per code of the widened int8 tiles, no widening). Turning packed int3 codes
// into fp4 costs more per code than widening them, so the GEMM never does it:
// the quantisers write activation codes as fp4, and weights are converted
// once (codes_to_fp4_kernel).
#include <algorithm>
#include <type_traits>

#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

namespace {

constexpr int kBK = 128;       // codes per k step (4 matrix-core steps of 32)
static_assert(kBK == 128, "the k step is written as four 32-code steps");
constexpr int kRowLds = 144;   // LDS bytes per row: 128 int8 + 16 pad (conflict-free 16-byte reads)

// Tile-internal format: int4 codes kept packed in LDS (256-code k steps),
// widened after the LDS read. Packed rows are the same bytes as for bits 4.
constexpr int kInt4Raw = 2;
static_assert(kInt4Raw != 3 && kInt4Raw != 4 && kInt4Raw != kFp4, "format ids must differ");

template <int BITS> struct Fmt;
template <> struct Fmt<4> {
    static constexpr int kGroupB = 16;   // packed bytes of 32 codes
    static constexpr int kShift = 8;     // (16 a)(16 w) = 256 a w
};
template <> struct Fmt<3> {
    static constexpr int kGroupB = 12;
    static constexpr int kShift = 10;    // (32 a)(32 w) = 1024 a w
};
template <> struct Fmt<kInt4Raw> {
    static constexpr int kGroupB = 16;   // packed bytes of 32 codes
    static constexpr int kShift = 8;     // widened as for bits 4: (16 a)(16 w)
};
template <> struct Fmt<kFp4> {
    static constexpr int kGroupB = 16;   // 32 nibbles
    static constexpr int kShift = 0;     // the matrix core multiplies the codes themselves
};

template <typename YT> __device__ __forceinline__ YT to_out(float v);
template <> __device__ __forceinline__ float to_out<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t to_out<uint16_t>(float v) {
    return static_cast<uint16_t>(pk_bf16(v, 0.0f));  // nearest even, one instruction
}
__device__ __forceinline__ float from_out(float v) { return v; }
__device__ __forceinline__ float from_out(uint16_t v) { return bf16_to_f32(v); }

// One group of 32 packed codes, as loaded from HBM.
template <int BITS> struct Group;
template <> struct Group<4> {
    v4u x;
    __device__ __forceinline__ void load(const uint8_t *p) { x = *reinterpret_cast<const v4u *>(p); }
    __device__ __forceinline__ void keep_if(bool ok) {
        x = v4u{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
    }
    // 32 int8 values (16 * code) in the order the matrix core consumes: lanes
    // of half 0 take bytes 0-15, half 1 bytes 16-31.
    __device__ __forceinline__ void widen(v4i &lo, v4i &hi) const {
        lo = unpack_int4x16(x[0], x[1]);
        hi = unpack_int4x16(x[2], x[3]);
    }
};
template <> struct Group<3> {
    uint32_t w0, w1, w2;
    __device__ __forceinline__ void load(const uint8_t *p) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
        w0 = q[0]; w1 = q[1]; w2 = q[2];
    }
    __device__ __forceinline__ void keep_if(bool ok) {
        w0 = ok ? w0 : 0u; w1 = ok ? w1 : 0u; w2 = ok ? w2 : 0u;
    }
    __device__ __forceinline__ void widen(v4i &lo, v4i &hi) const {
        lo = unpack_int3_half(w0, w1, w2, 0);
        hi = unpack_int3_half(w0, w1, w2, 1);
    }
};
template <> struct Group<kInt4Raw> {
    v4u x;
    __device__ __forceinline__ void load(const uint8_t *p) { x = *reinterpret_cast<const v4u *>(p); }
    __device__ __forceinline__ void keep_if(bool ok) {
        x = v4u{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
    }
};
template <> struct Group<kFp4> {
    v4u x;
    __device__ __forceinline__ void load(const uint8_t *p) { x = *reinterpret_cast<const v4u *>(p); }
    __device__ __forceinline__ void keep_if(bool ok) {
        x = v4u{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
    }
};

// Tile order. The hardware deals workgroups round-robin to the 8 XCDs
// (block b runs on XCD b % 8), each with its own L2. Block b is given a tile
// from a contiguous range owned by its XCD, and tiles are numbered channel
// tile major, so an XCD streams only its share of the weights and the
// workgroups resident on it at one time share weight tiles.
__device__ __forceinline__ int xcd_tile(int bid, int tiles) {
    constexpr int kXcd = 8;
    const int x = bid % kXcd, local = bid / kXcd;
    const int base = tiles / kXcd, rem = tiles % kXcd;
    return x * base + min(x, rem) + local;
}

// BM tokens x BN channels per workgroup, WM x WN waves, each wave
// (BM / WM) x (BN / WN) as TM x TN fragments of 32 x 32. Codes are widened to
// int8 once, on their way into LDS; the inner loop is 16-byte LDS reads
// straight into v_mfma_i32_32x32x32_i8. fp4 codes (BITS = kFp4) go into LDS
// as loaded, a k step is 256 codes (the same 128 LDS bytes per row) and each
// 16-byte read feeds v_mfma_scale_f32_32x32x64_f8f6f4; packed int4 codes
// (BITS = kInt4Raw) take the same LDS layout and each 16-byte read feeds two
// v_mfma_i32_32x32x32_i8 after widening.
template <int BITS, int BM, int BN, int WM, int WN, int P>
struct GemmTile {
    using F = Fmt<BITS>;
    static constexpr bool MX = BITS == kFp4;
    static constexpr bool RAW = MX || BITS == kInt4Raw;   // groups go into LDS as loaded
    using Acc = typename std::conditional<MX, v16f, v16i>::type;
    static constexpr int KB = RAW ? 2 * kBK : kBK;        // codes per k step
    static constexpr int GB = RAW ? 16 : 32;              // LDS bytes of one 32-code group
    static constexpr int NT = WM * WN * 64;
    static constexpr int GPR = KB / 32;                   // code groups per row per k step
    static constexpr int GROUPS = (BM + BN) * GPR;
    static constexpr int GPT = (GROUPS + NT - 1) / NT;    // groups per thread
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static constexpr int LDS_BYTES = 2 * (BM + BN) * kRowLds;

    // Whether every thread's i-th group lies in the A rows (0), the W rows (1)
    // or either (2); known at compile time for the shapes used.
    static constexpr int side(int i) {
        return NT * (i + 1) <= BM * GPR ? 0 : (NT * i >= BM * GPR ? 1 : 2);
    }

    // Main loop. FAST: the tile lies inside both matrices and K is a multiple
    // of KB, so loads need no clamping and no masking, and their addresses
    // are a per-thread 32-bit offset from a workgroup-uniform base.
    template <bool FAST>
    __device__ __forceinline__ static void run(uint8_t *lds, const uint8_t *A, const uint8_t *W, int n, int N,
                                               int K, int bm0, int bn0, Acc (&acc)[TM][TN]) {
        const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
        const int wm = wv / WN, wn = wv % WN;
        const int h = lane >> 5, l32 = lane & 31;
        const uint32_t rb = static_cast<uint32_t>(K) / 32 * F::kGroupB;  // packed row bytes
        const int nkt = (K + KB - 1) / KB;
        const uint8_t *abase = A + static_cast<size_t>(bm0) * rb;
        const uint8_t *wbase = W + static_cast<size_t>(bn0) * rb;

        uint32_t goff[GPT];
        int ldst[GPT], gk[GPT];
        bool gvalid[GPT], isa[GPT];
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int g = min(tid + NT * i, GROUPS - 1);  // threads past the end redo the last group
            const int row = g / GPR, part = g % GPR;      // LDS row: A rows first, then W rows
            isa[i] = row < BM;
            const int r = isa[i] ? row : row - BM;
            gvalid[i] = isa[i] ? bm0 + r < n : bn0 + r < N;
            goff[i] = (gvalid[i] ? static_cast<uint32_t>(r) : 0u) * rb + F::kGroupB * part;
            ldst[i] = row * kRowLds + GB * part;
            gk[i] = 32 * part;
        }
        auto src = [&](int i) -> const uint8_t * {
            if (side(i) == 0) return abase;
            if (side(i) == 1) return wbase;
            return isa[i] ? abase : wbase;
        };

        // P k steps of packed codes are in flight in registers (a ring of P
        // slots). In the main loop no load is behind a branch, so the compiler
        // keeps the newer slots' loads outstanding while it drains the oldest.
        // Outside FAST, addresses are clamped into the matrix and rows or k
        // groups outside it are zeroed when the slot is written to LDS.
        Group<BITS> stage[P][GPT];
        const int last_group_k = ((K - 1) / 32) * 32;    // k of the last 32-code group of a row
        auto load_tile = [&](int kt, Group<BITS> *st) {
            kt = min(kt, nkt - 1);
#pragma unroll
            for (int i = 0; i < GPT; ++i) {
                if constexpr (FAST) {
                    st[i].load(src(i) + goff[i] + static_cast<uint32_t>(kt) * (GPR * F::kGroupB));
                } else {
                    const int k = min(kt * KB + gk[i] - gk[i] % 32, last_group_k);
                    st[i].load(src(i) + goff[i] - (gk[i] / 32) * F::kGroupB + static_cast<uint32_t>(k / 32) * F::kGroupB);
                }
            }
        };
        // widen groups [i0, i1) of a slot (fp4: as they are) and write them
        // to an LDS buffer
        auto store_part = [&](int kt, uint8_t *buf, Group<BITS> *st, int i0, int i1) {
#pragma unroll
            for (int i = i0; i < i1; ++i) {
                if constexpr (!FAST) st[i].keep_if(gvalid[i] && kt * KB + gk[i] < K);
                if constexpr (RAW) {
                    *reinterpret_cast<v4u *>(buf + ldst[i]) = st[i].x;
                } else {
                    v4i lo, hi;
                    st[i].widen(lo, hi);
                    v4i *dst = reinterpret_cast<v4i *>(buf + ldst[i]);
                    dst[0] = lo;
                    dst[1] = hi;
                }
            }
        };

        const int arow = (wm * (BM / WM) + l32) * kRowLds + 16 * h;
        const int wrow = (BM + wn * (BN / WN) + l32) * kRowLds + 16 * h;
        // operands of one matrix-core step (32 int8 or 64 fp4 codes), double
        // buffered: step s + 1 is read from LDS while the matrix cores work on
        // step s
        v4i ao[2][TM], wo[2][TN];
        auto read_ops = [&](const uint8_t *lb, int s, int slot) {
#pragma unroll
            for (int i = 0; i < TM; ++i) ao[slot][i] = *reinterpret_cast<const v4i *>(lb + arow + 32 * i * kRowLds + 32 * s);
#pragma unroll
            for (int j = 0; j < TN; ++j) wo[slot][j] = *reinterpret_cast<const v4i *>(lb + wrow + 32 * j * kRowLds + 32 * s);
        };
        auto mfma = [&](int slot) {
            if constexpr (BITS == kInt4Raw) {
                // each 16-byte read holds one 32-code group: its low 8 bytes
                // feed the first multiply, its high 8 bytes the second (the
                // same split for both operands)
                v4i alo[TM], ahi[TM], blo[TN], bhi[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const v4i a = ao[slot][i];
                    alo[i] = unpack_int4x16(a[0], a[1]);
                    ahi[i] = unpack_int4x16(a[2], a[3]);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const v4i b = wo[slot][j];
                    blo[j] = unpack_int4x16(b[0], b[1]);
                    bhi[j] = unpack_int4x16(b[2], b[3]);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[i], blo[j], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[i], bhi[j], acc[i][j], 0, 0, 0);
                    }
                return;
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (MX) {
                        // fp4 (format 4) on both sides, block scale 2^1 (E8M0 128); an fp4
                        // operand is the low four registers
                        const v4i a = ao[slot][i], b = wo[slot][j];
                        const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
                        const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 0, 128,
                                                                                    0, 128);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[slot][i], wo[slot][j], acc[i][j], 0, 0, 0);
                    }
                }
        };
        // issue order inside one matrix-core step: multiplies alternate with
        // the LDS reads of the next step's operands
        auto interleave = [&]() {
#pragma unroll
            for (int q = 0; q < TM + TN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix-core op
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // One k step. LDS buffer kt & 1 holds step kt and the operands of its
        // first 32-code step are in slot 0. Slot u of the register ring is
        // refilled with step kt + P; step kt + 1 (slot u + 1) is widened into
        // the other buffer during the second and third 32-code steps. The
        // barrier comes before the last 32-code step, so its multiplies cover
        // the barrier and the LDS reads of step kt + 1's first operands.
        // Buffer reuse: the other buffer was last read before the previous
        // step's barrier, and this buffer is read only before this barrier.
        auto step = [&](int kt, int u) {
            const uint8_t *lb = lds + (kt & 1) * (LDS_BYTES / 2);
            uint8_t *nb = lds + ((kt + 1) & 1) * (LDS_BYTES / 2);
            load_tile(kt + P, stage[u]);
            read_ops(lb, 1, 1);
            mfma(0);
            interleave();
            read_ops(lb, 2, 0);
            store_part(kt + 1, nb, stage[(u + 1) % P], 0, GPT / 2);
            mfma(1);
            interleave();
            read_ops(lb, 3, 1);
            store_part(kt + 1, nb, stage[(u + 1) % P], GPT / 2, GPT);
            mfma(0);
            interleave();
            __syncthreads();
            read_ops(nb, 0, 0);
            mfma(1);
            interleave();
        };

#pragma unroll
        for (int u = 0; u < P; ++u) load_tile(u, stage[u]);
        store_part(0, lds, stage[0], 0, GPT);
        __syncthreads();
        read_ops(lds, 0, 0);
        int kt = 0;
        for (; kt + P <= nkt; kt += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) step(kt + u, u);
        }
#pragma unroll
        for (int u = 0; u < P - 1; ++u)
            if (kt + u < nkt) step(kt + u, u);
    }
};

// ---------------------------------------------------- decode-size batches
// One lane's packed codes of one 128-code k step of one row: lane half h takes
// codes [64h, 64h + 64) (groups 2h and 2h + 1) and matrix-core step s uses its
// 16-code block s. Activations and weights use the same order, so the dot
// products do not depend on it.
template <int BITS> struct Frag;
template <> struct Frag<4> {
    v4u x0, x1;
    __device__ __forceinline__ void load2(const uint8_t *g0, const uint8_t *g1) {
        x0 = *reinterpret_cast<const v4u *>(g0);
        x1 = *reinterpret_cast<const v4u *>(g1);
    }
    __device__ __forceinline__ v4i op(int s) const {
        return s == 0 ? unpack_int4x16(x0[0], x0[1])
                      : (s == 1 ? unpack_int4x16(x0[2], x0[3])
                                : (s == 2 ? unpack_int4x16(x1[0], x1[1]) : unpack_int4x16(x1[2], x1[3])));
    }
};
template <> struct Frag<3> {
    uint32_t w[6];
    __device__ __forceinline__ void load2(const uint8_t *g0, const uint8_t *g1) {  // 4-byte aligned
        const uint32_t *q0 = reinterpret_cast<const uint32_t *>(g0);
        const uint32_t *q1 = reinterpret_cast<const uint32_t *>(g1);
        w[0] = q0[0]; w[1] = q0[1]; w[2] = q0[2];
        w[3] = q1[0]; w[4] = q1[1]; w[5] = q1[2];
    }
    __device__ __forceinline__ v4i op(int s) const {
        const int g = s >> 1;
        return unpack_int3_half(w[3 * g], w[3 * g + 1], w[3 * g + 2], s & 1);
    }
};

// n <= 64 tokens: the weights are streamed once, so what counts is how many
// weight bytes are in flight. A workgroup owns 32 output channels and all
// tokens (TM fragments of 32); its NW waves split the k steps (wave w takes
// steps w, w + NW, ...), load their operands straight from global memory into
// registers in the matrix-core layout two steps ahead, and sum their partial
// accumulators through LDS at the end. No barrier inside the k loop.
template <int BITS, int TM, int NW, typename YT>
__global__ __launch_bounds__(NW * 64) void qgemv_kernel(const uint8_t *__restrict__ A, const float *__restrict__ sa,
                                                        int n, const uint8_t *__restrict__ W,
                                                        const float *__restrict__ sw, int N, int K,
                                                        YT *__restrict__ y, int64_t ld_y,
                                                        int32_t *__restrict__ acc_out, const YT *__restrict__ res,
                                                        int64_t ld_r) {
    using F = Fmt<BITS>;
    constexpr int KSTEP_B = kBK * BITS / 8;   // packed bytes of one k step of a row
    __shared__ int32_t red[NW][TM][16][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int h = lane >> 5, l32 = lane & 31;
    const int bn0 = blockIdx.x * 32;
    const uint32_t rb = static_cast<uint32_t>(K) * BITS / 8;
    const int nkt = (K + kBK - 1) / kBK;
    const uint8_t *wrow = W + static_cast<size_t>(min(bn0 + l32, N - 1)) * rb;
    const uint8_t *arow[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = A + static_cast<size_t>(min(32 * i + l32, n - 1)) * rb;

    Frag<BITS> fa[2][TM], fw[2];
    // groups past the row end read the row's first group (in bounds); the
    // weight operand of such a group is zeroed before use
    auto load_step = [&](int kt, int slot) {
        kt = min(kt, nkt - 1);
        const int k0 = kt * kBK + 64 * h;
        const uint32_t off0 = k0 < K ? static_cast<uint32_t>(kt) * KSTEP_B + h * (KSTEP_B / 2) : 0u;
        const uint32_t off1 = k0 + 32 < K ? static_cast<uint32_t>(kt) * KSTEP_B + h * (KSTEP_B / 2) + F::kGroupB : 0u;
        fw[slot].load2(wrow + off0, wrow + off1);
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[slot][i].load2(arow[i] + off0, arow[i] + off1);
    };
    v16i acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0;
    auto compute = [&](int kt, int slot) {
        if (kt >= nkt) return;
#pragma unroll
        for (int s = 0; s < kBK / 32; ++s) {
            v4i wo = fw[slot].op(s);
            if (kt * kBK + 64 * h + 32 * (s >> 1) >= K) wo = v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[slot][i].op(s), wo, acc[i], 0, 0, 0);
        }
    };
    load_step(w, 0);
    load_step(w + NW, 1);
    for (int kt = w; kt < nkt; kt += 2 * NW) {
        compute(kt, 0);
        load_step(kt + 2 * NW, 0);
        compute(kt + NW, 1);
        load_step(kt + 3 * NW, 1);
    }

    // sum the waves' partial accumulators (fixed order) and write the outputs
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[w][i][v][lane] = acc[i][v];
    __syncthreads();
    for (int e = threadIdx.x; e < TM * 16 * 64; e += NW * 64) {
        const int i = e / 1024, v = (e / 64) % 16, ln = e % 64;
        int a = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) a += red[ww][i][v][ln];
        const int tok = 32 * i + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
        const int ch = bn0 + (ln & 31);
        if (tok < n && ch < N) {
            a >>= F::kShift;
            float val = (static_cast<float>(a) * sa[tok]) * sw[ch];
            if (res != nullptr) val += from_out(res[static_cast<int64_t>(tok) * ld_r + ch]);
            y[static_cast<int64_t>(tok) * ld_y + ch] = to_out<YT>(val);
            if (acc_out != nullptr) acc_out[static_cast<int64_t>(tok) * N + ch] = a;
        }
    }
}

// n <= 64 tokens, 16 output channels per workgroup on v_mfma_i32_16x16x64_i8
// (A = activations, rows = tokens; B = weights, columns = channels). A
// 256-code k step is split over the lane quarters: lane quarter q takes codes
// [64q, 64q + 64) (groups 2q and 2q + 1) and matrix-core step s its 16-code
// block s, the same order for both operands. NW waves take k steps w, w + NW,
// ... with operands loaded straight into registers D steps ahead and sum
// their accumulators through LDS at the end in a fixed order.
template <int BITS, int TB, int NW, typename YT, int D = 2>
__global__ __launch_bounds__(NW * 64) void qgemv16_kernel(const uint8_t *__restrict__ A, const float *__restrict__ sa,
                                                          int n, const uint8_t *__restrict__ W,
                                                          const float *__restrict__ sw, int N, int K,
                                                          YT *__restrict__ y, int64_t ld_y,
                                                          int32_t *__restrict__ acc_out, const YT *__restrict__ res,
                                                          int64_t ld_r) {
    using F = Fmt<BITS>;
    constexpr int KSB = 256 * BITS / 8;     // packed bytes of one 256-code step of a row
    __shared__ int32_t red[NW][TB][4][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int q = lane >> 4, c16 = lane & 15;
    const int bn0 = blockIdx.x * 16;
    const uint32_t rb = static_cast<uint32_t>(K) * BITS / 8;
    const int nkt = (K + 255) / 256;
    const uint8_t *wrow = W + static_cast<size_t>(bn0 + c16) * rb;
    const uint8_t *arow[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) arow[i] = A + static_cast<size_t>(min(16 * i + c16, n - 1)) * rb;

    Frag<BITS> fa[D][TB], fw[D];
    // groups past the row end read the row's first group (in bounds); the
    // weight operand of such a group is zeroed before use
    auto load_step = [&](int kt, int slot) {
        kt = min(kt, nkt - 1);
        const int k0 = kt * 256 + 64 * q;
        const uint32_t base = static_cast<uint32_t>(kt) * KSB + q * (KSB / 4);
        const uint32_t off0 = k0 < K ? base : 0u;
        const uint32_t off1 = k0 + 32 < K ? base + F::kGroupB : 0u;
        fw[slot].load2(wrow + off0, wrow + off1);
#pragma unroll
        for (int i = 0; i < TB; ++i) fa[slot][i].load2(arow[i] + off0, arow[i] + off1);
    };
    v4i acc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) acc[i] = v4i{0, 0, 0, 0};
    auto compute = [&](int kt, int slot) {
        if (kt >= nkt) return;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v4i wo = fw[slot].op(s);
            if (kt * 256 + 64 * q + 32 * (s >> 1) >= K) wo = v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < TB; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[slot][i].op(s), wo, acc[i], 0, 0, 0);
        }
    };
    // a ring of D register slots: slot u holds k step kt + u NW while the
    // steps before it are multiplied (steps past the end reload the last one)
#pragma unroll
    for (int u = 0; u < D; ++u) load_step(w + u * NW, u);
    for (int kt = w; kt < nkt; kt += D * NW) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            compute(kt + u * NW, u);
            load_step(kt + (u + D) * NW, u);
        }
    }

    // sum the waves' partial accumulators (fixed order) and write the outputs:
    // lane l, register v holds token 16 i + 4 (l / 16) + v, channel l % 16
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][i][v][lane] = acc[i][v];
    __syncthreads();
    for (int e = threadIdx.x; e < TB * 4 * 64; e += NW * 64) {
        const int i = e / 256, v = (e / 64) % 4, ln = e % 64;
        int a = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) a += red[ww][i][v][ln];
        const int tok = 16 * i + 4 * (ln >> 4) + v;
        const int ch = bn0 + (ln & 15);
        if (tok < n) {
            a >>= F::kShift;
            float val = (static_cast<float>(a) * sa[tok]) * sw[ch];
            if (res != nullptr) val += from_out(res[static_cast<int64_t>(tok) * ld_r + ch]);
            y[static_cast<int64_t>(tok) * ld_y + ch] = to_out<YT>(val);
            if (acc_out != nullptr) acc_out[static_cast<int64_t>(tok) * N + ch] = a;
        }
    }
}

template <int BITS, int TB, int NW, typename YT, int D = 2>
hipError_t launch_gemv16(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw, int64_t N,
                         int64_t K, void *y, int64_t ld_y, int32_t *acc_out, const void *res, int64_t ld_r,
                         hipStream_t s) {
    if (!grid_fits(N / 16, NW * 64)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((qgemv16_kernel<BITS, TB, NW, YT, D>), dim3(static_cast<unsigned>(N / 16)), dim3(NW * 64), 0,
                       s, a, sa, static_cast<int>(n), w, sw, static_cast<int>(N), static_cast<int>(K),
                       static_cast<YT *>(y), ld_y, acc_out, static_cast<const YT *>(res), ld_r);
    return hipGetLastError();
}

template <int BITS, int TM, typename YT, int NW = 8>
hipError_t launch_gemv(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw, int64_t N,
                       int64_t K, void *y, int64_t ld_y, int32_t *acc_out, const void *res, int64_t ld_r,
                       hipStream_t s) {
    if (!grid_fits((N + 31) / 32, NW * 64)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((qgemv_kernel<BITS, TM, NW, YT>), dim3(static_cast<unsigned>((N + 31) / 32)), dim3(NW * 64), 0,
                       s, a, sa, static_cast<int>(n), w, sw, static_cast<int>(N), static_cast<int>(K),
                       static_cast<YT *>(y), ld_y, acc_out, static_cast<const YT *>(res), ld_r);
    return hipGetLastError();
}

template <int BITS, int BM, int BN, int WM, int WN, int P, typename YT>
__global__ __launch_bounds__(WM * WN * 64) void qgemm_kernel(const uint8_t *__restrict__ A,
                                                             const float *__restrict__ sa, int n,
                                                             const uint8_t *__restrict__ W,
                                                             const float *__restrict__ sw, int N, int K,
                                                             YT *__restrict__ y, int64_t ld_y,
                                                             int32_t *__restrict__ acc_out,
                                                             const YT *__restrict__ res, int64_t ld_r) {
    using T = GemmTile<BITS, BM, BN, WM, WN, P>;
    constexpr int SH = Fmt<BITS>::kShift;  // scale of the int8 path's sums
    constexpr int TM = T::TM, TN = T::TN;
    __shared__ __attribute__((aligned(16))) uint8_t lds[T::LDS_BYTES];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv / WN, wn = wv % WN;
    const int h = lane >> 5, l32 = lane & 31;
    const int mt = (n + BM - 1) / BM;
    const int tiles = mt * ((N + BN - 1) / BN);
    const int tile = xcd_tile(blockIdx.x, tiles);
    const int bm0 = (tile % mt) * BM;
    const int bn0 = (tile / mt) * BN;

    typename T::Acc accm[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) accm[i][j][v] = 0;

    if (bm0 + BM <= n && bn0 + BN <= N && K % T::KB == 0)
        T::template run<true>(lds, A, W, n, N, K, bm0, bn0, accm);
    else
        T::template run<false>(lds, A, W, n, N, K, bm0, bn0, accm);
    // (the fp4 path's float32 sums are exact integers)
    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = static_cast<int>(accm[i][j][v]);

    // epilogue: lane holds channel l32 of each fragment and tokens 8(v/4) + 4h + v%4
    constexpr int OS = BN + 8;  // bf16 row stride of the output tile in LDS
    constexpr int CPR = BN / 8;  // 16-byte chunks per row of the tile
    const bool staged = sizeof(YT) == 2 && acc_out == nullptr && ld_y % 8 == 0 &&
                        (reinterpret_cast<uintptr_t>(y) & 15) == 0 && BM * OS * 2 <= T::LDS_BYTES &&
                        (res == nullptr || (ld_r % 8 == 0 && (reinterpret_cast<uintptr_t>(res) & 15) == 0));
    if (staged) {
        // bf16 tile through LDS, then 16-byte row-contiguous stores
        uint16_t *ot = reinterpret_cast<uint16_t *>(lds);
        // the scales of this lane's 16 * TM tokens, loaded once for all its channels
        float sat[TM][16];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tl = wm * (BM / WM) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                sat[i][v] = bm0 + tl < n ? sa[bm0 + tl] : 0.0f;
            }
        __syncthreads();  // every wave is done with the operand tiles
        if (res != nullptr) {
            // the residual tile, read with the same 16-byte row-contiguous
            // accesses into the slots its sums will take (in place: this tile
            // is read entirely before any of it is written)
            for (int c = threadIdx.x; c < BM * CPR; c += WM * WN * 64) {
                const int r = c / CPR, q = c % CPR;
                if (bm0 + r < n && bn0 + 8 * q < N)
                    *reinterpret_cast<v4u *>(ot + r * OS + 8 * q) =
                        *reinterpret_cast<const v4u *>(res + static_cast<int64_t>(bm0 + r) * ld_r + bn0 + 8 * q);
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int cl = wn * (BN / WN) + 32 * j + l32;
            const float swj = bn0 + cl < N ? sw[bn0 + cl] : 0.0f;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int tl = wm * (BM / WM) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                    float val = (static_cast<float>(acc[i][j][v] >> SH) * sat[i][v]) * swj;
                    if (res != nullptr) val += bf16_to_f32(ot[tl * OS + cl]);
                    ot[tl * OS + cl] = to_out<uint16_t>(val);
                }
            }
        }
        __syncthreads();
        for (int c = threadIdx.x; c < BM * CPR; c += WM * WN * 64) {
            const int r = c / CPR, q = c % CPR;
            if (bm0 + r < n && bn0 + 8 * q < N)
                *reinterpret_cast<v4u *>(y + static_cast<int64_t>(bm0 + r) * ld_y + bn0 + 8 * q) =
                    *reinterpret_cast<const v4u *>(ot + r * OS + 8 * q);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int ch = bn0 + wn * (BN / WN) + 32 * j + l32;
        const bool cvalid = ch < N;
        const float swj = cvalid ? sw[ch] : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tok = bm0 + wm * (BM / WM) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (cvalid && tok < n) {
                    const int a = acc[i][j][v] >> SH;
                    float val = (static_cast<float>(a) * sa[tok]) * swj;
                    if (res != nullptr) val += from_out(res[static_cast<int64_t>(tok) * ld_r + ch]);
                    y[static_cast<int64_t>(tok) * ld_y + ch] = to_out<YT>(val);
                    if (acc_out != nullptr) acc_out[static_cast<int64_t>(tok) * N + ch] = a;
                }
            }
        }
    }
}

template <int BITS, int BM, int BN, int WM, int WN, typename YT, int P = 2>
hipError_t launch_t(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw, int64_t N,
                    int64_t K, void *y, int64_t ld_y, int32_t *acc_out, const void *res, int64_t ld_r, hipStream_t s) {
    const int64_t mt = (n + BM - 1) / BM, nt = (N + BN - 1) / BN;
    if (!grid_fits(mt * nt, WM * WN * 64)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((qgemm_kernel<BITS, BM, BN, WM, WN, P, YT>), dim3(static_cast<unsigned>(mt * nt)),
                       dim3(WM * WN * 64), 0, s, a, sa, static_cast<int>(n), w, sw, static_cast<int>(N),
                       static_cast<int>(K), static_cast<YT *>(y), ld_y, acc_out, static_cast<const YT *>(res), ld_r);
    return hipGetLastError();
}

// Tile shape by problem size (measured on MI355X): 256 tokens x 128, 192 or
// 256 channels with 8 waves on the layer shapes, whichever needs the least
// time in whole rounds of workgroups over the compute units (wider tiles read
// fewer LDS bytes per multiply); 128 x 128 for mid-size batches; narrow or
// k-split kernels for decode-size batches.
template <int BITS, typename YT>
hipError_t launch_b(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw, int64_t N,
                    int64_t K, void *y, int64_t ld_y, int32_t *acc_out, const void *res, int64_t ld_r, hipStream_t s) {
    const int64_t cus = device_cus();
    // int4 on the 32 x 32, 64 x 64 and 256 x 128 tiles: packed in LDS (see the
    // top of the file; e.g. 64 tokens, q|k|v: 11.4 against 13.6 us; 32 tokens,
    // gate|up: 11.8 against 15.7 us); the wider tiles keep the widened form
    constexpr int PK = BITS == 4 ? kInt4Raw : BITS;
    if constexpr (BITS == kFp4) {
        // the fp4 operands have no decode-size kernels of their own: narrow tiles
        if (n <= 32) return launch_t<BITS, 32, 32, 1, 1, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
        if (n <= 64) return launch_t<BITS, 64, 64, 2, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
    } else {
        // decode-size batches stream the weights once
        const int64_t gemv_wgs = (N + 31) / 32;
        // up to 16 tokens, or up to 64 while 16-channel workgroups fit the CUs in
        // one round: 16-channel workgroups on the 16 x 16 x 64 matrix core (more
        // workgroups streaming the weights; measured faster than the kernels
        // below for 1 and 8 tokens on every layer shape and for 64 tokens at
        // N = 4096; slower at 64 tokens for N = 12288 and 22016, where every
        // workgroup re-reads all 64 activation rows)
        // long k: more k steps in flight (up to 16 tokens: 4 waves with a
        // 3-step ring, e.g. 1 token at K = 11008: 6.5 against 7.5 us for 8
        // waves with 2; more tokens: 8 waves with 2). A layer whose 16-channel
        // workgroups fit the CUs in one round takes 8 waves as well (o, 4096 x
        // 4096: 1 token 4.7 against 5.4 us, 8 tokens 5.0 against 5.7, 64
        // tokens 9.2 against 9.9; the widest layers keep 4: gate|up, 22016 x
        // 4096, 8 tokens 14.7 against 16.2 us).
        if (n <= 16 || (n <= 64 && N / 16 <= cus)) {
            const bool deep = K >= 8192;
            const bool wide = deep || N / 16 <= cus;   // 8 waves per workgroup
            switch ((n + 15) / 16) {
            case 1: return deep ? launch_gemv16<BITS, 1, 4, YT, 3>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s)
                                : (wide ? launch_gemv16<BITS, 1, 8, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s)
                                        : launch_gemv16<BITS, 1, 4, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s));
            case 2: return wide ? launch_gemv16<BITS, 2, 8, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s)
                                : launch_gemv16<BITS, 2, 4, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
            case 3: return wide ? launch_gemv16<BITS, 3, 8, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s)
                                : launch_gemv16<BITS, 3, 4, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
            default: return wide ? launch_gemv16<BITS, 4, 8, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s)
                                 : launch_gemv16<BITS, 4, 4, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
            }
        }
        // 17-64 tokens on the wider layers: 32-channel workgroups while they fit
        // the CUs in one round (up to 48 tokens), else 32 x 32 tiles up to 32
        // tokens and 64 x 64 tiles beyond (64 x 64 tiles halve the re-reads of
        // the activation rows of 64 x 32 tiles: q|k|v at 64 tokens 13.1 against
        // 15.2 us). Measured as graph replays: 32-channel workgroups in two
        // rounds are the slowest choice (q|k|v, 12288 x 4096, 32 tokens: 14.7
        // against 11.4 us on 32 x 32 tiles); in one round the fastest up to 48
        // tokens (6144 x 4096, 24 tokens: 8.0 against 12.2 us).
        if (n <= 32) {
            if (gemv_wgs <= cus) return launch_gemv<BITS, 1, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
            return launch_t<PK, 32, 32, 1, 1, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
        }
        if (n <= 64) {
            if (gemv_wgs <= cus && n <= 48)
                return launch_gemv<BITS, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
            return launch_t<PK, 64, 64, 2, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
        }
    }
    const int64_t mt = (n + 255) / 256;
    if (n < 256 || mt * ((N + 127) / 128) < 200)
        return launch_t<BITS, 128, 128, 2, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
    // 256-token tiles, 128, 192 or 256 channels wide: rounds of workgroups
    // over the CUs times the tile's relative time (tile width over its
    // measured relative efficiency 1 : 1.09 : 1.17)
    auto cost = [&](int64_t bn, int64_t eff100) {
        const int64_t rounds = (mt * ((N + bn - 1) / bn) + cus - 1) / cus;
        return rounds * bn * 100 * 117 / eff100;
    };
    const int64_t c128 = cost(128, 100), c192 = cost(192, 109), c256 = cost(256, 117);
    if (c256 < c128 && c256 <= c192)
        return launch_t<BITS, 256, 256, 4, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
    if (c192 < c128)
        return launch_t<BITS, 256, 192, 4, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
    return launch_t<PK, 256, 128, 4, 2, YT>(a, sa, n, w, sw, N, K, y, ld_y, acc_out, res, ld_r, s);
}

// ------------------------------------------------- int3 codes -> fp4 codes
// Per byte of a word: a 3-bit two's complement code u in bits 7-5 and another
// in bits 4-2 -> two e2m1 nibbles of u / 2 (sign in bit 3, |u| in bits 1-0).
// |u| keeps u's low bit; its second bit flips where the sign and the low bit
// are both set (-1 -> 1, -3 -> 3, -2 -> 2).
__device__ __forceinline__ uint32_t fp4_pair(uint32_t x) {
    const uint32_t t = x & (x >> 2);  // sign AND low bit: bit 5 (high code), bit 2 (low code)
    const uint32_t base = (x & 0x80808080u) | ((x >> 1) & 0x38383838u) | ((x >> 2) & 0x03030303u);
    return base ^ ((t & 0x20202020u) | ((t >> 1) & 0x02020202u));
}

// One thread per 32-code group: 12 bytes of int3 codes (words w0, w1, w2) ->
// 16 bytes of fp4. Word i of the output takes slots 2i (high nibbles) and
// 2i + 1 (low nibbles); slots 6 and 7 are first gathered into the bit
// positions of slots 0 and 1.
__global__ __launch_bounds__(256) void codes_to_fp4_kernel(const uint32_t *__restrict__ in, v4u *__restrict__ out,
                                                           int64_t groups) {
    for (int64_t g = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; g < groups;
         g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const uint32_t w0 = in[3 * g], w1 = in[3 * g + 1], w2 = in[3 * g + 2];
        const uint32_t x3 = ((w2 << 6) & 0x80808080u) | ((w0 << 5) & 0x60606060u) | ((w2 << 4) & 0x10101010u) |
                            ((w1 << 2) & 0x0C0C0C0Cu);
        out[g] = v4u{fp4_pair(w0), fp4_pair(w1), fp4_pair(w2), fp4_pair(x3)};
    }
}

}  // namespace

hipError_t launch_codes_to_fp4(const uint8_t *codes, int64_t rows, int64_t k, uint8_t *out, hipStream_t s) {
    const int64_t groups = rows * (k / 32);
    const int64_t blocks = std::min<int64_t>((groups + 255) / 256, static_cast<int64_t>(device_cus()) * 16);
    hipLaunchKernelGGL(codes_to_fp4_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t *>(codes), reinterpret_cast<v4u *>(out), groups);
    return hipGetLastError();
}

hipError_t launch_qgemm(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw,
                        int64_t n_out, int64_t k, int bits, void *y, int y_dtype, int64_t ld_y,
                        int32_t *acc_out, const void *res, int64_t ld_r, void *ws, hipStream_t s) {
    (void)ws;   // see qgemm_workspace_bytes
    if (bits == kFp4) {
        if (y_dtype == 1) return launch_b<kFp4, uint16_t>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, res, ld_r, s);
        return launch_b<kFp4, float>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, res, ld_r, s);
    }
    if (bits == 4) {
        if (y_dtype == 1) return launch_b<4, uint16_t>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, res, ld_r, s);
        return launch_b<4, float>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, res, ld_r, s);
    }
    if (y_dtype == 1) return launch_b<3, uint16_t>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, res, ld_r, s);
    return launch_b<3, float>(a, sa, n, w, sw, n_out, k, y, ld_y, acc_out, res, ld_r, s);
}

size_t qgemm_workspace_bytes(int64_t n, int64_t n_out, int64_t k, int bits) {
    // no GEMM kernel splits its k range over workgroups: a split whose partial
    // sums meet through device memory needs device-scope release and acquire
    // fences, which write back or invalidate the whole L2 of an XCD, and
    // measured 3-4 times slower than the single-workgroup decode kernels
    (void)n; (void)n_out; (void)k; (void)bits;
    return 0;
}

}  // namespace rsq
