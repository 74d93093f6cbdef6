// Offline fusion of a rotation into a linear's weight (ReSpinQuant's offline
// weight fusion, zh 2.2 - e.g. W~ = R^T W R - and fr 2A, W~ = W R): with the
// linear's input in a basis rotated by R (h~ = h R), y = h W^T = h~ (W R)^T;
// an output basis R' gives R'^T W. One launch applies one side:
//   right: out = W R      (W: n x k, R: k x k)
//   left:  out = R^T W    (R: n x n)
// float32 operands, float64 products and sums (a float32 product is exact in
// float64), one rounding to float32 per output. Not on the per-token path:
// it runs once per model, so a plain LDS-tiled float64 FMA GEMM serves.
#include "rsq_device.h"
#include "rsq_internal.h"

namespace rsq {

namespace {

constexpr int kTile = 64;   // outputs per side of a workgroup tile
constexpr int kStep = 16;   // inner-dimension step

// C (rows x cols) = A (rows x inner) B (inner x cols). LEFT: A(m, i) = R[i][m]
// (R is rows x rows, inner = rows), B = W; right: A = W (inner = cols),
// B = R. 256 threads, each 4 x 4 outputs.
template <bool LEFT>
__global__ __launch_bounds__(256) void rotate_kernel(const float *__restrict__ W, const float *__restrict__ R,
                                                     float *__restrict__ out, int rows, int cols) {
    __shared__ double as[kStep][kTile + 1];
    __shared__ double bs[kStep][kTile + 1];
    const int inner = LEFT ? rows : cols;
    const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int k0 = 0; k0 < inner; k0 += kStep) {
        // each thread stages 4 elements of each tile (16 x 64), zero outside the matrices
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + 256 * q;
            const int kk = e / kTile, mm = e % kTile;      // A tile element (kk, mm): A(m0 + mm, k0 + kk)
            const int m = m0 + mm, k = k0 + kk;
            float a = 0.0f;
            if (m < rows && k < inner) a = LEFT ? R[static_cast<size_t>(k) * rows + m] : W[static_cast<size_t>(m) * cols + k];
            as[kk][mm] = static_cast<double>(a);
            const int n = n0 + mm;                          // B tile element (kk, mm): B(k0 + kk, n0 + mm)
            float b = 0.0f;
            if (n < cols && k < inner) b = LEFT ? W[static_cast<size_t>(k) * cols + n] : R[static_cast<size_t>(k) * cols + n];
            bs[kk][mm] = static_cast<double>(b);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kStep; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = as[kk][4 * ty + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = bs[kk][4 * tx + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * ty + i;
        if (m >= rows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + 4 * tx + j;
            if (n < cols) out[static_cast<size_t>(m) * cols + n] = static_cast<float>(acc[i][j]);
        }
    }
}

}  // namespace

hipError_t launch_rotate_weight(const float *W, int64_t n, int64_t k, const float *R, bool left, float *out,
                                hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((k + kTile - 1) / kTile), static_cast<unsigned>((n + kTile - 1) / kTile));
    if (left)
        hipLaunchKernelGGL(rotate_kernel<true>, grid, dim3(256), 0, s, W, R, out, static_cast<int>(n), static_cast<int>(k));
    else
        hipLaunchKernelGGL(rotate_kernel<false>, grid, dim3(256), 0, s, W, R, out, static_cast<int>(n), static_cast<int>(k));
    return hipGetLastError();
}

}  // namespace rsq
