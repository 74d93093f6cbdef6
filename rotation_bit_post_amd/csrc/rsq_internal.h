// Internal launcher interface between the C ABI (rsq_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rsq {

// r rounded up to a multiple of 32 (the matrix-core K step of the reprojection).
inline int rank_pad(int r) { return (r + 31) / 32 * 32; }

// Bytes of a prepared site: U and V = U M^T, each as bf16 hi + lo, d x r_pad
// (parts U hi, V hi, U lo, V lo).
inline size_t site_bytes(int64_t d, int r) { return static_cast<size_t>(d) * rank_pad(r) * 2 * 2 * 2; }

// Code formats (the launchers' `bits`): packed int4 (4), packed int3 (3), and
// 3-bit codes held as fp4 e2m1 nibbles (kFp4).
constexpr int kFp4 = 1;

// Most waves in a correction workgroup.
constexpr int kCorrectMaxWaves = 8;

// Waves per workgroup and 32-column chunks per wave of the correction kernel
// for width d: the fewest chunks per wave (1, 2, 4, ... 32; at most 16 for a
// float32 residual, whose slice of 32 chunks does not fit in registers) that
// split d / 32 evenly over at most kCorrectMaxWaves waves. False if none does.
inline bool correct_geometry(int64_t d, bool f32, int *waves, int *chunks_per_wave) {
    if (d <= 0 || d % 32) return false;
    const int64_t nch = d / 32;
    for (int cpw : {1, 2, 4, 8, 16, 32}) {
        if (f32 && cpw > 16) break;
        if (nch % cpw == 0 && nch / cpw <= kCorrectMaxWaves) {
            *waves = static_cast<int>(nch / cpw);
            *chunks_per_wave = cpw;
            return true;
        }
    }
    return false;
}

// Whether `blocks` workgroups of `threads` threads fit one dispatch: fewer
// than 2^31 workgroups and fewer than 2^32 threads in all. Launchers return
// hipErrorInvalidConfiguration otherwise, rather than let a grid size wrap.
inline bool grid_fits(int64_t blocks, int64_t threads) {
    return blocks > 0 && blocks < (int64_t{1} << 31) && blocks * threads < (int64_t{1} << 32);
}

// Compute units of the current device (cached per device).
int device_cus();

hipError_t launch_site_prepare(const float *U, const float *M, int d, int r, void *site, hipStream_t s);

// h_dtype: 0 float32, 1 bfloat16. quant: also RMSNorm + quantise + pack
// (bits: 4, 3 or kFp4, the format of the codes written). ws: device scratch
// of at least correct_workspace_bytes(n, d) bytes, or NULL when that is 0.
hipError_t launch_correct(const void *h_in, void *h_out, int h_dtype, int64_t n, int d, int64_t ld_h,
                          const void *site, int r, bool quant, const float *norm_w, float eps, int bits,
                          uint8_t *codes, float *scales, void *ws, hipStream_t s);

// Scratch bytes the quantising correction needs for n tokens of width d
// (0: no correction kernel exchanges data between workgroups).
size_t correct_workspace_bytes(int64_t n, int64_t d);

hipError_t launch_quant(const void *x, int x_dtype, int64_t n, int k, int64_t ld_x, bool norm,
                        const float *norm_w, float eps, int bits, uint8_t *codes, float *scales,
                        hipStream_t s);

// Offline weight fusion: out = W R (R: k x k) or, with left, out = R^T W (R: n x n);
// W and out: n x k row-major float32.
hipError_t launch_rotate_weight(const float *W, int64_t n, int64_t k, const float *R, bool left, float *out,
                                hipStream_t s);

// Packed int3 rows (k codes each) -> fp4 rows (k / 2 bytes each).
hipError_t launch_codes_to_fp4(const uint8_t *codes, int64_t rows, int64_t k, uint8_t *out, hipStream_t s);

// res: NULL, or n rows of n_out values of the output type (stride ld_r) added
// to the dequantised result before its rounding. bits: 4, 3 or kFp4. ws:
// device scratch of at least qgemm_workspace_bytes(n, n_out, k, bits) bytes,
// or NULL when that is 0.
hipError_t launch_qgemm(const uint8_t *a, const float *sa, int64_t n, const uint8_t *w, const float *sw,
                        int64_t n_out, int64_t k, int bits, void *y, int y_dtype, int64_t ld_y,
                        int32_t *acc_out, const void *res, int64_t ld_r, void *ws, hipStream_t s);

// Scratch bytes of the GEMM launch for these sizes (0: no GEMM kernel splits
// its k range over workgroups). bits: 4, 3 or kFp4.
size_t qgemm_workspace_bytes(int64_t n, int64_t n_out, int64_t k, int bits);

}  // namespace rsq
