/*
 * rsq.h - C ABI of the ReSpinQuant online path on AMD Instinct MI355X (gfx950).
 *
 * Sources: the five gist.science summaries of "ReSpinQuant: Efficient
 * Layer-Wise LLM Quantization via Subspace Residual Rotation Approximation"
 * (arXiv 2604.11080), cited as <language> <section>, e.g. "zh 2.2" is the
 * Chinese summary, technical section 2.2.
 *
 * Conventions (every entry point):
 *  - Memory: the caller owns all memory. Pointers named "host" are host
 *    pointers; every other pointer is a device pointer on the current HIP
 *    device, at least 16-byte aligned. The library allocates nothing.
 *  - Workspace: the entry points that take `workspace, workspace_bytes` may
 *    need device scratch (for work split over workgroups whose partial
 *    results meet through device memory), sized by the matching
 *    rsq_*_workspace_bytes query for the same sizes; a result of 0 means
 *    NULL, 0 may be passed. In this version every query returns 0: each
 *    kernel keeps its exchanges inside a workgroup. A workspace, where one is
 *    needed, is zero-filled before its first use and left zero-filled by
 *    every call; calls that share one must not run concurrently (enqueue
 *    them on one stream). Too small a workspace is RSQ_ERR_WORKSPACE.
 *  - Execution: work is enqueued on `stream` (a hipStream_t; NULL is the
 *    null stream) and the call returns without waiting. Device faults show
 *    at the caller's next synchronisation.
 *  - Errors: the return value is an rsq_status. Arguments are checked before
 *    anything is enqueued; on an error nothing is enqueued and no output is
 *    touched. rsq_last_error() gives a message for the calling thread's last
 *    failed call.
 *  - Rows: a "row" is one token. Row strides (ld_*) are in elements.
 *  - Codes: signed 4-bit codes in [-7, 7] or 3-bit codes in [-3, 3], packed
 *    per row, K codes in rsq_packed_row_bytes(K, bits) bytes:
 *      int4: byte j holds code 2j in bits 0-3 and code 2j+1 in bits 4-7
 *            (two's complement nibbles);
 *      int3: groups of 32 codes in 12 bytes = words w0, w1, w2 (4 bytes each,
 *            byte lane b = byte b of a word); code i of a group (3-bit two's
 *            complement u, slot j = i/4, lane b = i%4) sits at
 *              slots 0,2,4: bits 5-7 of lane b of word j/2;
 *              slots 1,3,5: bits 2-4 of lane b of word (j-1)/2;
 *              slot 6: u bits 0-1 -> bits 0-1 of lane b of w0, u bit 2 -> bit 1 of lane b of w2;
 *              slot 7: u bits 0-1 -> bits 0-1 of lane b of w1, u bit 2 -> bit 0 of lane b of w2.
 *  - fp4 codes (rsq_codes_to_fp4, rsq_qgemm_fp4, bits = 3 | RSQ_FP4): 3-bit codes c in [-3, 3]
 *    held as OCP MX fp4 (e2m1) values c / 2, one nibble each (bit 3 the sign,
 *    bits 0-1 |c|, bit 2 zero), k / 2 bytes per row; each group of 32 codes
 *    (the int3 group above) takes 16 bytes: byte 4i + b (i, b < 4) holds
 *    code 8i + b in bits 4-7 and code 8i + 4 + b in bits 0-3.
 *  - Sizes: d and k multiples of 32; n_out a multiple of 32; n >= 0 (n = 0
 *    enqueues nothing); 1 <= r <= 64; bits 3 or 4 (or 3 | RSQ_FP4, below). Upper limits (beyond
 *    them RSQ_ERR_UNSUPPORTED): k <= 65536 for the GEMMs (the int32
 *    accumulator bound), k <= 32768 for rsq_quant_act (one row in the
 *    registers of at most four waves); for the correction d / 32 must split
 *    into at most 8 waves of 1, 2, 4, 8, 16 or 32 column chunks (at most 16
 *    for a float32 residual), i.e. d <= 8192 (4096 for float32). A launch that
 *    would need more than 2^31 workgroups or 2^32 threads in one dispatch
 *    is refused with RSQ_ERR_HIP instead of being enqueued (buffers of such
 *    sizes exceed a device's memory; rsq_layer_fused may then already have
 *    enqueued its correction).
 */
#ifndef RSQ_H
#define RSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RSQ_OK = 0,
    RSQ_ERR_INVALID_ARG = 1,   /* null pointer, negative or inconsistent size, misalignment */
    RSQ_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels handle (e.g. r > 64) */
    RSQ_ERR_WORKSPACE = 3,     /* workspace NULL, misaligned or smaller than its query */
    RSQ_ERR_HIP = 4            /* the HIP runtime refused a launch or a query */
} rsq_status;

typedef enum { RSQ_F32 = 0, RSQ_BF16 = 1 } rsq_dtype;

/* rsq_quant_act flags */
#define RSQ_QA_RMSNORM 1u

/* OR'ed into bits = 3 (bits = 3 | RSQ_FP4): the 3-bit codes are read or
 * written in the fp4 layout instead of the packed int3 one: the codes that
 * rsq_quant_act, rsq_correct_quant and rsq_layer_fused write, and the
 * activation and weight codes that rsq_qgemm, rsq_qgemm_residual and
 * rsq_layer_fused read (rsq_packed_row_bytes gives k / 2). */
#define RSQ_FP4 0x100

#define RSQ_MAX_RANK 64

/* Library version (major*10000 + minor*100 + patch). */
int rsq_version(void);
/* Static string naming a status code. */
const char *rsq_status_str(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char *rsq_last_error(void);

/* Bytes of one packed row of k codes (0 if k or bits is invalid; bits 3,
 * 4 or 3 | RSQ_FP4). */
size_t rsq_packed_row_bytes(int64_t k, int bits);

/* Workspace bytes (see Conventions) of rsq_qgemm, rsq_qgemm_residual and
 * rsq_qgemm_fp4 (bits 3 | RSQ_FP4) for n tokens, n_out channels and k codes;
 * of rsq_correct_quant for n tokens of width d; of rsq_layer_fused for both
 * its stages. 0 if no kernel for these sizes needs scratch, or if a size is
 * invalid (the call then reports the invalid size). */
size_t rsq_qgemm_workspace_bytes(int64_t n, int64_t n_out, int64_t k, int bits);
size_t rsq_correct_workspace_bytes(int64_t n, int64_t d);
size_t rsq_layer_workspace_bytes(int64_t n, int64_t d, int64_t n_out, int bits);

/*
 * Correction site (offline, once per model). The pages apply, per residual
 * junction, y = Q^T x, then M = R_sub - I_r inside the r-dimensional
 * subspace, then add Q (M y) back (zh 2.2 steps 1-3; fr 2C), with Q the top-r
 * singular vectors of dT = T - I, T = R_out^T R_in (it 2C; nl 2C; fr 2C).
 * For a row vector h this is h' = h + ((h U) M) U^T.
 *
 * rsq_site_prepare turns U (d x r, row-major float32) and M (r x r, row-major
 * float32) into the device layout the kernels read: U and V = U M^T, each
 * split into a bfloat16 high part and a bfloat16 remainder, laid out as the
 * matrix-core operands, r padded to a multiple of 32 with zeros.
 * site: device buffer of rsq_site_bytes(d, r) bytes, written by this call.
 */
size_t rsq_site_bytes(int64_t d, int r);
rsq_status rsq_site_prepare(const float *U, const float *M, int64_t d, int r,
                            void *site, void *stream);

/*
 * Subspace residual rotation (zh 2.2 steps 1-3; fr 2C):
 *   h_out[t, :] = h_in[t, :] + ((h_in[t, :] U) M) U^T   for t < n,
 * computed with float32 accumulation and rounded once (nearest-even) to
 * h_dtype. h_in, h_out: n rows of d elements, row stride ld_h (>= d).
 * h_in == h_out (in place) is allowed; any other overlap is not.
 */
rsq_status rsq_subspace_correct(const void *h_in, void *h_out, int h_dtype,
                                int64_t n, int64_t d, int64_t ld_h,
                                const void *site, int r, void *stream);

/*
 * Per-token symmetric activation quantisation (the A4 / A3 settings of
 * zh 4 and fr 4), with optional RMSNorm first (flags & RSQ_QA_RMSNORM):
 *   inv   = float32(1 / sqrt(mean_k(x^2) + eps))       (sum of squares in float64;
 *           within a few float32 ulps of the exact sum: the summation
 *           order is the kernel's)
 *   a     = (x * inv) * w    (float32; w = norm_w, or 1 if norm_w is NULL);
 *           without the flag a = x
 *   s     = max_k |a| / qmax                           (qmax = 7 for bits 4, 3 for 3-bit codes)
 *   q     = clamp(rint(a / s), -qmax, qmax)             (float32 quotient, ties to even)
 *   a zero row gives s = 0 and q = 0.
 * x: n rows of k elements (x_dtype), stride ld_x. codes: n rows of
 * rsq_packed_row_bytes(k, bits) bytes, contiguous. scales: n floats.
 * norm_w: k floats or NULL.
 */
rsq_status rsq_quant_act(const void *x, int x_dtype, int64_t n, int64_t k, int64_t ld_x,
                         unsigned flags, const float *norm_w, float eps, int bits,
                         uint8_t *codes, float *scales, void *stream);

/*
 * Correction, RMSNorm and quantisation in one pass over the residual:
 * rsq_subspace_correct followed by rsq_quant_act(RSQ_QA_RMSNORM) on the
 * rounded h_out (the norm reads h_out as stored). h_out is identical to
 * rsq_subspace_correct's; the sum of squares is taken in another order
 * (bfloat16 squares summed by 8 in float32, exactly per product, then in
 * float64), so scales may differ from rsq_quant_act's by a few ulps and codes
 * only where a / s lies that close to a rounding tie. Batches too small to
 * fill the GPU with token blocks (not in place) run as two launches: the
 * correction split over the columns, then rsq_quant_act's kernel on the
 * stored rows (its results exactly).
 * h_in, h_out: contiguous rows (stride d). workspace: see Conventions
 * (rsq_correct_workspace_bytes).
 */
rsq_status rsq_correct_quant(const void *h_in, void *h_out, int h_dtype, int64_t n, int64_t d,
                             const void *site, int r, const float *norm_w, float eps, int bits,
                             uint8_t *codes, float *scales, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Quantised linear with per-token and per-channel dequantisation (W4A4 /
 * W3A3; a standard linear once the rotations are fused, zh 2.2 and nl 2A):
 *   acc[t, j] = sum_k a[t, k] * w[j, k]                   (exact int32)
 *   y[t, j]   = (float32(acc[t, j]) * a_scales[t]) * w_scales[j]   (float32), then y_dtype
 * a_codes: n packed rows of k codes; w_codes: n_out packed rows of k codes.
 * y: n rows, stride ld_y (>= n_out). acc_out: NULL, or n x n_out int32
 * (contiguous) that receives the raw accumulators. workspace: see
 * Conventions (rsq_qgemm_workspace_bytes; also for rsq_qgemm_residual and
 * rsq_qgemm_fp4).
 */
rsq_status rsq_qgemm(const uint8_t *a_codes, const float *a_scales, int64_t n,
                     const uint8_t *w_codes, const float *w_scales, int64_t n_out,
                     int64_t k, int bits, void *y, int y_dtype, int64_t ld_y,
                     int32_t *acc_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Quantised linear plus a residual: the residual adds around the attention
 * and FFN blocks, whose junctions carry the corrections (zh 2.1; fr 2B),
 * fused into the linear's output so that the o_proj and down_proj results
 * land on the residual stream in one pass:
 *   y[t, j] = y_dtype(v + float32(residual[t, j])),  v as in rsq_qgemm (float32)
 * residual: n rows of n_out values of y_dtype, row stride ld_r; it may be y
 * itself (in place, ld_r == ld_y); any other overlap is an error.
 */
rsq_status rsq_qgemm_residual(const uint8_t *a_codes, const float *a_scales, int64_t n,
                              const uint8_t *w_codes, const float *w_scales, int64_t n_out,
                              int64_t k, int bits, const void *residual, int64_t ld_r,
                              void *y, int y_dtype, int64_t ld_y, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * 3-bit codes in another layout for the fp4 matrix cores: each of `rows`
 * packed int3 rows of k codes (rsq_packed_row_bytes(k, 3) bytes, contiguous)
 * becomes a row of k / 2 bytes of fp4 codes (contiguous), the same values.
 * Weights are converted once; activation codes once per linear (a pass over
 * the codes, far cheaper than converting inside the GEMM, where every
 * workgroup of a row of tiles would convert the same codes again).
 * codes, fp4: 16-byte aligned, not overlapping.
 */
rsq_status rsq_codes_to_fp4(const uint8_t *codes, int64_t rows, int64_t k, uint8_t *fp4, void *stream);

/*
 * The W3A3 quantised linear (zh 4 and fr 4; the linear of zh 2.2 and nl 2A)
 * on fp4 codes: rsq_qgemm (bits 3) and, with residual non-NULL,
 * rsq_qgemm_residual, on the same codes in the fp4 layout; y and acc_out
 * are identical to theirs. The matrix cores multiply c_a / 2 by c_w / 2 with
 * a block scale of 2 on each side, so every product is c_a c_w exactly and
 * every partial sum an integer below 2^24, exact in their float32
 * accumulation.
 * a_fp4: n rows of k / 2 bytes; w_fp4: n_out rows of k / 2 bytes.
 * residual: NULL, or as in rsq_qgemm_residual (stride ld_r; may be y).
 * acc_out: NULL, or n x n_out int32 (contiguous).
 */
rsq_status rsq_qgemm_fp4(const uint8_t *a_fp4, const float *a_scales, int64_t n, const uint8_t *w_fp4,
                         const float *w_scales, int64_t n_out, int64_t k, const void *residual, int64_t ld_r, void *y,
                         int y_dtype, int64_t ld_y, int32_t *acc_out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Offline weight fusion (once per model, not per token): the pages fuse each
 * block's rotations into its weights offline (zh 2.2, offline weight fusion,
 * e.g. W~ = R^T W R; fr 2A, W~ = W R). For a linear y = h W^T whose input h
 * lives in a basis rotated by R (h~ = h R), y = h~ (W R)^T; an output kept in
 * a basis R' takes R'^T on the left. One call applies one side:
 *   side RSQ_ROTATE_RIGHT: W_out = W R      (R: k x k)
 *   side RSQ_ROTATE_LEFT:  W_out = R^T W    (R: n_out x n_out)
 * W, W_out: n_out x k row-major float32; R row-major float32. Products and
 * sums in float64, each output rounded once to float32. n_out and k multiples
 * of 32, at most 2^20; W_out must not overlap W or R.
 */
#define RSQ_ROTATE_RIGHT 0
#define RSQ_ROTATE_LEFT 1
rsq_status rsq_rotate_weight(const float *W, int64_t n_out, int64_t k, const float *R, int side, float *W_out,
                             void *stream);

/*
 * One correction site feeding its quantised linear: rsq_correct_quant then
 * rsq_qgemm on its codes. Writes h_out, codes, scales and y (stride n_out).
 * workspace: see Conventions (rsq_layer_workspace_bytes; the two stages run
 * one after the other and share it).
 */
rsq_status rsq_layer_fused(const void *h_in, void *h_out, int h_dtype, int64_t n, int64_t d,
                           const void *site, int r, const float *norm_w, float eps, int bits,
                           uint8_t *codes, float *scales,
                           const uint8_t *w_codes, const float *w_scales, int64_t n_out,
                           void *y, int y_dtype, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RSQ_H */
