// C ABI: argument checks, dispatch to the kernels, error reporting.
// Every check runs before anything is enqueued; a failed check leaves all
// outputs untouched.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/rsq.h"
#include "rsq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

rsq_status fail(rsq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

rsq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return RSQ_OK;
    return fail(RSQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int dt) { return dt == RSQ_F32 || dt == RSQ_BF16; }
size_t dtype_size(int dt) { return dt == RSQ_BF16 ? 2 : 4; }

#define RSQ_CHECK(cond, st, ...) \
    do {                          \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

rsq_status check_site(int64_t d, int r) {
    RSQ_CHECK(d > 0 && d % 32 == 0, RSQ_ERR_INVALID_ARG, "d = %lld must be a positive multiple of 32", (long long)d);
    RSQ_CHECK(r >= 1, RSQ_ERR_INVALID_ARG, "r = %d must be >= 1", r);
    RSQ_CHECK(r <= RSQ_MAX_RANK, RSQ_ERR_UNSUPPORTED, "r = %d exceeds the supported maximum %d", r, RSQ_MAX_RANK);
    RSQ_CHECK(r <= d, RSQ_ERR_INVALID_ARG, "r = %d exceeds d = %lld", r, (long long)d);
    RSQ_CHECK(d <= (1 << 20), RSQ_ERR_UNSUPPORTED, "d = %lld too large", (long long)d);
    int nw = 0, cpw = 0;
    RSQ_CHECK(rsq::correct_geometry(d, false, &nw, &cpw), RSQ_ERR_UNSUPPORTED,
              "d = %lld: d/32 must split into at most 8 waves of 1, 2, 4, 8, 16 or 32 chunks", (long long)d);
    return RSQ_OK;
}

rsq_status check_bits(int bits) {
    RSQ_CHECK(bits == 3 || bits == 4 || bits == (3 | RSQ_FP4), RSQ_ERR_INVALID_ARG,
              "bits = %d must be 3, 4 or 3 | RSQ_FP4", bits);
    return RSQ_OK;
}

// The launchers' code format for a checked `bits`.
int code_format(int bits) { return bits == (3 | RSQ_FP4) ? rsq::kFp4 : bits; }

// A workspace of `have` bytes at ws for a launch that needs `need`.
rsq_status check_workspace(size_t need, const void *ws, size_t have) {
    if (need == 0) return RSQ_OK;
    RSQ_CHECK(ws != nullptr && aligned16(ws), RSQ_ERR_WORKSPACE,
              "a workspace of %zu bytes is needed (non-null, 16-byte aligned)", need);
    RSQ_CHECK(have >= need, RSQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", have, need);
    return RSQ_OK;
}

rsq_status check_norm_w(const float *norm_w) {
    RSQ_CHECK(norm_w == nullptr || aligned16(norm_w), RSQ_ERR_INVALID_ARG, "norm_w must be 16-byte aligned");
    return RSQ_OK;
}

bool gemm_sizes_ok(int64_t n, int64_t n_out, int64_t k) {
    return n >= 0 && n <= 0x7fffffff && n_out > 0 && n_out % 32 == 0 && n_out <= 0x7fffffff && k > 0 &&
           k % 32 == 0 && k <= 65536;
}

rsq_status check_correct_args(const void *h_in, const void *h_out, int h_dtype, int64_t n, int64_t d, int64_t ld_h,
                              const void *site, int r) {
    RSQ_CHECK(dtype_ok(h_dtype), RSQ_ERR_INVALID_ARG, "h_dtype = %d is not RSQ_F32 or RSQ_BF16", h_dtype);
    RSQ_CHECK(n >= 0, RSQ_ERR_INVALID_ARG, "n = %lld is negative", (long long)n);
    rsq_status st = check_site(d, r);
    if (st != RSQ_OK) return st;
    int nw = 0, cpw = 0;
    RSQ_CHECK(h_dtype != RSQ_F32 || rsq::correct_geometry(d, true, &nw, &cpw), RSQ_ERR_UNSUPPORTED,
              "d = %lld: a float32 residual needs d/32 split into at most 8 waves of at most 16 chunks",
              (long long)d);
    RSQ_CHECK(ld_h >= d, RSQ_ERR_INVALID_ARG, "ld_h = %lld < d = %lld", (long long)ld_h, (long long)d);
    RSQ_CHECK((ld_h * (int64_t)dtype_size(h_dtype)) % 16 == 0, RSQ_ERR_INVALID_ARG,
              "row stride of %lld bytes is not a multiple of 16", (long long)(ld_h * (int64_t)dtype_size(h_dtype)));
    if (n == 0) return RSQ_OK;
    RSQ_CHECK(h_in && h_out && site, RSQ_ERR_INVALID_ARG, "null pointer (h_in, h_out or site)");
    RSQ_CHECK(aligned16(h_in) && aligned16(h_out) && aligned16(site), RSQ_ERR_INVALID_ARG,
              "h_in, h_out and site must be 16-byte aligned");
    if (h_in != h_out) {
        const char *a = static_cast<const char *>(h_in), *b = static_cast<const char *>(h_out);
        const size_t span = static_cast<size_t>((n - 1) * ld_h + d) * dtype_size(h_dtype);
        RSQ_CHECK(a + span <= b || b + span <= a, RSQ_ERR_INVALID_ARG, "h_in and h_out overlap without being equal");
    }
    return RSQ_OK;
}

rsq_status check_quant_out(int64_t n, int64_t k, int bits, const uint8_t *codes, const float *scales) {
    rsq_status st = check_bits(bits);
    if (st != RSQ_OK) return st;
    if (n == 0) return RSQ_OK;
    RSQ_CHECK(codes && scales, RSQ_ERR_INVALID_ARG, "null pointer (codes or scales)");
    RSQ_CHECK(aligned16(codes) && aligned16(scales), RSQ_ERR_INVALID_ARG, "codes and scales must be 16-byte aligned");
    (void)k;
    return RSQ_OK;
}

// Sizes, pointers and alignment shared by the quantised linears.
rsq_status check_gemm(int64_t n, int64_t n_out, int64_t k, int y_dtype, int64_t ld_y, const void *a_codes,
                      const float *a_scales, const void *w_codes, const float *w_scales, const void *y) {
    RSQ_CHECK(dtype_ok(y_dtype), RSQ_ERR_INVALID_ARG, "y_dtype = %d is not RSQ_F32 or RSQ_BF16", y_dtype);
    RSQ_CHECK(n >= 0, RSQ_ERR_INVALID_ARG, "n = %lld is negative", (long long)n);
    RSQ_CHECK(n_out > 0 && n_out % 32 == 0, RSQ_ERR_INVALID_ARG, "n_out = %lld must be a positive multiple of 32", (long long)n_out);
    RSQ_CHECK(k > 0 && k % 32 == 0, RSQ_ERR_INVALID_ARG, "k = %lld must be a positive multiple of 32", (long long)k);
    RSQ_CHECK(k <= 65536, RSQ_ERR_UNSUPPORTED, "k = %lld exceeds 65536 (int32 accumulator bound)", (long long)k);
    RSQ_CHECK(ld_y >= n_out, RSQ_ERR_INVALID_ARG, "ld_y = %lld < n_out = %lld", (long long)ld_y, (long long)n_out);
    RSQ_CHECK(n <= 0x7fffffff && n_out <= 0x7fffffff, RSQ_ERR_UNSUPPORTED, "size too large");
    if (n == 0) return RSQ_OK;
    RSQ_CHECK(a_codes && a_scales && w_codes && w_scales && y, RSQ_ERR_INVALID_ARG, "null pointer");
    RSQ_CHECK(aligned16(a_codes) && aligned16(w_codes) && aligned16(a_scales) && aligned16(w_scales) && aligned16(y),
              RSQ_ERR_INVALID_ARG, "operands must be 16-byte aligned");
    return RSQ_OK;
}

// The residual of a linear: n rows of n_out values of y_dtype, stride ld_r;
// either y itself (same stride) or disjoint from it.
rsq_status check_residual(int64_t n, int64_t n_out, int y_dtype, const void *residual, int64_t ld_r, const void *y,
                          int64_t ld_y) {
    RSQ_CHECK(ld_r >= n_out, RSQ_ERR_INVALID_ARG, "ld_r = %lld < n_out = %lld", (long long)ld_r, (long long)n_out);
    if (n == 0) return RSQ_OK;
    RSQ_CHECK(residual != nullptr && aligned16(residual), RSQ_ERR_INVALID_ARG, "residual must be non-null and 16-byte aligned");
    if (residual != y) {
        const size_t es = dtype_size(y_dtype);
        const char *a = static_cast<const char *>(residual), *b = static_cast<const char *>(y);
        const size_t span_r = static_cast<size_t>((n - 1) * ld_r + n_out) * es;
        const size_t span_y = static_cast<size_t>((n - 1) * ld_y + n_out) * es;
        RSQ_CHECK(a + span_r <= b || b + span_y <= a, RSQ_ERR_INVALID_ARG,
                  "residual and y overlap without being the same buffer");
    } else {
        RSQ_CHECK(ld_r == ld_y, RSQ_ERR_INVALID_ARG, "in place (residual == y) needs ld_r == ld_y");
    }
    return RSQ_OK;
}

}  // namespace

extern "C" {

int rsq_version(void) { return 200; }

const char *rsq_status_str(int status) {
    switch (status) {
        case RSQ_OK: return "RSQ_OK";
        case RSQ_ERR_INVALID_ARG: return "RSQ_ERR_INVALID_ARG";
        case RSQ_ERR_UNSUPPORTED: return "RSQ_ERR_UNSUPPORTED";
        case RSQ_ERR_WORKSPACE: return "RSQ_ERR_WORKSPACE";
        case RSQ_ERR_HIP: return "RSQ_ERR_HIP";
        default: return "RSQ_UNKNOWN_STATUS";
    }
}

const char *rsq_last_error(void) { return g_last_error; }

size_t rsq_packed_row_bytes(int64_t k, int bits) {
    if (k <= 0 || k % 32) return 0;
    if (bits == 4 || bits == (3 | RSQ_FP4)) return static_cast<size_t>(k) / 2;
    if (bits == 3) return static_cast<size_t>(k) * 3 / 8;
    return 0;
}

size_t rsq_qgemm_workspace_bytes(int64_t n, int64_t n_out, int64_t k, int bits) {
    if (!gemm_sizes_ok(n, n_out, k) || rsq_packed_row_bytes(k, bits) == 0 || n == 0) return 0;
    return rsq::qgemm_workspace_bytes(n, n_out, k, code_format(bits));
}

size_t rsq_correct_workspace_bytes(int64_t n, int64_t d) {
    int nw = 0, cpw = 0;
    if (n <= 0 || n > 0x7fffffff || !rsq::correct_geometry(d, false, &nw, &cpw)) return 0;
    return rsq::correct_workspace_bytes(n, d);
}

size_t rsq_layer_workspace_bytes(int64_t n, int64_t d, int64_t n_out, int bits) {
    const size_t a = rsq_correct_workspace_bytes(n, d), b = rsq_qgemm_workspace_bytes(n, n_out, d, bits);
    return a > b ? a : b;
}

size_t rsq_site_bytes(int64_t d, int r) {
    if (d <= 0 || d % 32 || r < 1 || r > RSQ_MAX_RANK || r > d) return 0;
    return rsq::site_bytes(d, r);
}

rsq_status rsq_site_prepare(const float *U, const float *M, int64_t d, int r, void *site, void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_site(d, r);
    if (st != RSQ_OK) return st;
    RSQ_CHECK(U && M && site, RSQ_ERR_INVALID_ARG, "null pointer (U, M or site)");
    RSQ_CHECK(aligned16(site), RSQ_ERR_INVALID_ARG, "site must be 16-byte aligned");
    return hip_status(rsq::launch_site_prepare(U, M, static_cast<int>(d), r, site, static_cast<hipStream_t>(stream)),
                      "rsq_site_prepare launch");
}

rsq_status rsq_subspace_correct(const void *h_in, void *h_out, int h_dtype, int64_t n, int64_t d, int64_t ld_h,
                                const void *site, int r, void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_correct_args(h_in, h_out, h_dtype, n, d, ld_h, site, r);
    if (st != RSQ_OK || n == 0) return st;
    return hip_status(rsq::launch_correct(h_in, h_out, h_dtype, n, static_cast<int>(d), ld_h, site, r, false,
                                          nullptr, 0.0f, 4, nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream)),
                      "rsq_subspace_correct launch");
}

rsq_status rsq_quant_act(const void *x, int x_dtype, int64_t n, int64_t k, int64_t ld_x, unsigned flags,
                         const float *norm_w, float eps, int bits, uint8_t *codes, float *scales, void *stream) {
    g_last_error[0] = 0;
    RSQ_CHECK(dtype_ok(x_dtype), RSQ_ERR_INVALID_ARG, "x_dtype = %d is not RSQ_F32 or RSQ_BF16", x_dtype);
    RSQ_CHECK(n >= 0, RSQ_ERR_INVALID_ARG, "n = %lld is negative", (long long)n);
    RSQ_CHECK(k > 0 && k % 32 == 0, RSQ_ERR_INVALID_ARG, "k = %lld must be a positive multiple of 32", (long long)k);
    RSQ_CHECK(k <= 32768, RSQ_ERR_UNSUPPORTED, "k = %lld exceeds 32768", (long long)k);
    RSQ_CHECK(ld_x >= k, RSQ_ERR_INVALID_ARG, "ld_x = %lld < k = %lld", (long long)ld_x, (long long)k);
    RSQ_CHECK((ld_x * (int64_t)dtype_size(x_dtype)) % 16 == 0, RSQ_ERR_INVALID_ARG, "row stride not a multiple of 16 bytes");
    RSQ_CHECK((flags & ~RSQ_QA_RMSNORM) == 0, RSQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    RSQ_CHECK(!(flags & RSQ_QA_RMSNORM) || eps >= 0.0f, RSQ_ERR_INVALID_ARG, "eps must be >= 0");
    RSQ_CHECK(n <= 0x7fffffff, RSQ_ERR_UNSUPPORTED, "n too large");
    rsq_status st = check_quant_out(n, k, bits, codes, scales);
    if (st != RSQ_OK) return st;
    st = check_norm_w(norm_w);
    if (st != RSQ_OK || n == 0) return st;
    RSQ_CHECK(x != nullptr && aligned16(x), RSQ_ERR_INVALID_ARG, "x must be non-null and 16-byte aligned");
    return hip_status(rsq::launch_quant(x, x_dtype, n, static_cast<int>(k), ld_x, (flags & RSQ_QA_RMSNORM) != 0,
                                        norm_w, eps, code_format(bits), codes, scales, static_cast<hipStream_t>(stream)),
                      "rsq_quant_act launch");
}

rsq_status rsq_correct_quant(const void *h_in, void *h_out, int h_dtype, int64_t n, int64_t d, const void *site,
                             int r, const float *norm_w, float eps, int bits, uint8_t *codes, float *scales,
                             void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_correct_args(h_in, h_out, h_dtype, n, d, d, site, r);
    if (st != RSQ_OK) return st;
    RSQ_CHECK(eps >= 0.0f, RSQ_ERR_INVALID_ARG, "eps must be >= 0");
    st = check_quant_out(n, d, bits, codes, scales);
    if (st != RSQ_OK) return st;
    st = check_norm_w(norm_w);
    if (st != RSQ_OK || n == 0) return st;
    st = check_workspace(rsq::correct_workspace_bytes(n, d), workspace, workspace_bytes);
    if (st != RSQ_OK) return st;
    return hip_status(rsq::launch_correct(h_in, h_out, h_dtype, n, static_cast<int>(d), d, site, r, true, norm_w,
                                          eps, code_format(bits), codes, scales, workspace,
                                          static_cast<hipStream_t>(stream)),
                      "rsq_correct_quant launch");
}

rsq_status rsq_qgemm(const uint8_t *a_codes, const float *a_scales, int64_t n, const uint8_t *w_codes,
                     const float *w_scales, int64_t n_out, int64_t k, int bits, void *y, int y_dtype, int64_t ld_y,
                     int32_t *acc_out, void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_bits(bits);
    if (st != RSQ_OK) return st;
    st = check_gemm(n, n_out, k, y_dtype, ld_y, a_codes, a_scales, w_codes, w_scales, y);
    if (st != RSQ_OK || n == 0) return st;
    RSQ_CHECK(acc_out == nullptr || aligned16(acc_out), RSQ_ERR_INVALID_ARG, "acc_out must be 16-byte aligned");
    st = check_workspace(rsq::qgemm_workspace_bytes(n, n_out, k, code_format(bits)), workspace, workspace_bytes);
    if (st != RSQ_OK) return st;
    return hip_status(rsq::launch_qgemm(a_codes, a_scales, n, w_codes, w_scales, n_out, k, code_format(bits), y,
                                        y_dtype, ld_y, acc_out, nullptr, 0, workspace,
                                        static_cast<hipStream_t>(stream)),
                      "rsq_qgemm launch");
}

rsq_status rsq_qgemm_residual(const uint8_t *a_codes, const float *a_scales, int64_t n, const uint8_t *w_codes,
                              const float *w_scales, int64_t n_out, int64_t k, int bits, const void *residual,
                              int64_t ld_r, void *y, int y_dtype, int64_t ld_y, void *workspace,
                              size_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_bits(bits);
    if (st != RSQ_OK) return st;
    st = check_gemm(n, n_out, k, y_dtype, ld_y, a_codes, a_scales, w_codes, w_scales, y);
    if (st != RSQ_OK) return st;
    st = check_residual(n, n_out, y_dtype, residual, ld_r, y, ld_y);
    if (st != RSQ_OK || n == 0) return st;
    st = check_workspace(rsq::qgemm_workspace_bytes(n, n_out, k, code_format(bits)), workspace, workspace_bytes);
    if (st != RSQ_OK) return st;
    return hip_status(rsq::launch_qgemm(a_codes, a_scales, n, w_codes, w_scales, n_out, k, code_format(bits), y,
                                        y_dtype, ld_y, nullptr, residual, ld_r, workspace,
                                        static_cast<hipStream_t>(stream)),
                      "rsq_qgemm_residual launch");
}

rsq_status rsq_codes_to_fp4(const uint8_t *codes, int64_t rows, int64_t k, uint8_t *fp4, void *stream) {
    g_last_error[0] = 0;
    RSQ_CHECK(rows >= 0, RSQ_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
    RSQ_CHECK(k > 0 && k % 32 == 0, RSQ_ERR_INVALID_ARG, "k = %lld must be a positive multiple of 32", (long long)k);
    RSQ_CHECK(rows <= ((int64_t)1 << 40) / k, RSQ_ERR_UNSUPPORTED, "rows x k too large");
    if (rows == 0) return RSQ_OK;
    RSQ_CHECK(codes && fp4, RSQ_ERR_INVALID_ARG, "null pointer (codes or fp4)");
    RSQ_CHECK(aligned16(codes) && aligned16(fp4), RSQ_ERR_INVALID_ARG, "codes and fp4 must be 16-byte aligned");
    const char *a = reinterpret_cast<const char *>(codes), *b = reinterpret_cast<const char *>(fp4);
    const size_t span_in = static_cast<size_t>(rows) * (static_cast<size_t>(k) * 3 / 8);
    const size_t span_out = static_cast<size_t>(rows) * (static_cast<size_t>(k) / 2);
    RSQ_CHECK(a + span_in <= b || b + span_out <= a, RSQ_ERR_INVALID_ARG, "codes and fp4 overlap");
    return hip_status(rsq::launch_codes_to_fp4(codes, rows, k, fp4, static_cast<hipStream_t>(stream)),
                      "rsq_codes_to_fp4 launch");
}

rsq_status rsq_qgemm_fp4(const uint8_t *a_fp4, const float *a_scales, int64_t n, const uint8_t *w_fp4,
                         const float *w_scales, int64_t n_out, int64_t k, const void *residual, int64_t ld_r, void *y,
                         int y_dtype, int64_t ld_y, int32_t *acc_out, void *workspace, size_t workspace_bytes,
                         void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_gemm(n, n_out, k, y_dtype, ld_y, a_fp4, a_scales, w_fp4, w_scales, y);
    if (st != RSQ_OK) return st;
    if (residual != nullptr) {
        st = check_residual(n, n_out, y_dtype, residual, ld_r, y, ld_y);
        if (st != RSQ_OK) return st;
    }
    if (n == 0) return RSQ_OK;
    RSQ_CHECK(acc_out == nullptr || aligned16(acc_out), RSQ_ERR_INVALID_ARG, "acc_out must be 16-byte aligned");
    st = check_workspace(rsq::qgemm_workspace_bytes(n, n_out, k, rsq::kFp4), workspace, workspace_bytes);
    if (st != RSQ_OK) return st;
    return hip_status(rsq::launch_qgemm(a_fp4, a_scales, n, w_fp4, w_scales, n_out, k, rsq::kFp4, y, y_dtype, ld_y,
                                        acc_out, residual, residual != nullptr ? ld_r : 0, workspace,
                                        static_cast<hipStream_t>(stream)),
                      "rsq_qgemm_fp4 launch");
}

rsq_status rsq_rotate_weight(const float *W, int64_t n_out, int64_t k, const float *R, int side, float *W_out,
                             void *stream) {
    g_last_error[0] = 0;
    RSQ_CHECK(side == RSQ_ROTATE_RIGHT || side == RSQ_ROTATE_LEFT, RSQ_ERR_INVALID_ARG,
              "side = %d is not RSQ_ROTATE_RIGHT or RSQ_ROTATE_LEFT", side);
    RSQ_CHECK(n_out > 0 && n_out % 32 == 0 && k > 0 && k % 32 == 0, RSQ_ERR_INVALID_ARG,
              "n_out = %lld and k = %lld must be positive multiples of 32", (long long)n_out, (long long)k);
    RSQ_CHECK(n_out <= (1 << 20) && k <= (1 << 20), RSQ_ERR_UNSUPPORTED, "n_out or k above 2^20");
    RSQ_CHECK(W && R && W_out, RSQ_ERR_INVALID_ARG, "null pointer (W, R or W_out)");
    RSQ_CHECK(aligned16(W) && aligned16(R) && aligned16(W_out), RSQ_ERR_INVALID_ARG,
              "W, R and W_out must be 16-byte aligned");
    const int64_t rd = side == RSQ_ROTATE_RIGHT ? k : n_out;
    const char *w0 = reinterpret_cast<const char *>(W), *r0 = reinterpret_cast<const char *>(R);
    const char *o0 = reinterpret_cast<const char *>(W_out);
    const size_t wb = static_cast<size_t>(n_out) * k * 4, rb = static_cast<size_t>(rd) * rd * 4;
    RSQ_CHECK((o0 + wb <= w0 || w0 + wb <= o0) && (o0 + wb <= r0 || r0 + rb <= o0), RSQ_ERR_INVALID_ARG,
              "W_out overlaps W or R");
    return hip_status(rsq::launch_rotate_weight(W, n_out, k, R, side == RSQ_ROTATE_LEFT, W_out,
                                                static_cast<hipStream_t>(stream)),
                      "rsq_rotate_weight launch");
}

rsq_status rsq_layer_fused(const void *h_in, void *h_out, int h_dtype, int64_t n, int64_t d, const void *site, int r,
                           const float *norm_w, float eps, int bits, uint8_t *codes, float *scales,
                           const uint8_t *w_codes, const float *w_scales, int64_t n_out, void *y, int y_dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    rsq_status st = check_correct_args(h_in, h_out, h_dtype, n, d, d, site, r);
    if (st != RSQ_OK) return st;
    st = check_quant_out(n, d, bits, codes, scales);
    if (st != RSQ_OK) return st;
    st = check_norm_w(norm_w);
    if (st != RSQ_OK) return st;
    RSQ_CHECK(eps >= 0.0f, RSQ_ERR_INVALID_ARG, "eps must be >= 0");
    RSQ_CHECK(dtype_ok(y_dtype), RSQ_ERR_INVALID_ARG, "y_dtype = %d is not RSQ_F32 or RSQ_BF16", y_dtype);
    RSQ_CHECK(n_out > 0 && n_out % 32 == 0, RSQ_ERR_INVALID_ARG, "n_out = %lld must be a positive multiple of 32", (long long)n_out);
    RSQ_CHECK(d <= 65536, RSQ_ERR_UNSUPPORTED, "d = %lld exceeds 65536", (long long)d);
    if (n == 0) return RSQ_OK;
    RSQ_CHECK(w_codes && w_scales && y, RSQ_ERR_INVALID_ARG, "null pointer (w_codes, w_scales or y)");
    RSQ_CHECK(aligned16(w_codes) && aligned16(w_scales) && aligned16(y), RSQ_ERR_INVALID_ARG, "operands must be 16-byte aligned");
    // the two stages run one after the other on the stream: one workspace serves both
    const size_t need_c = rsq::correct_workspace_bytes(n, d);
    const size_t need_g = rsq::qgemm_workspace_bytes(n, n_out, d, code_format(bits));
    st = check_workspace(need_c > need_g ? need_c : need_g, workspace, workspace_bytes);
    if (st != RSQ_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(rsq::launch_correct(h_in, h_out, h_dtype, n, static_cast<int>(d), d, site, r, true, norm_w, eps,
                                        code_format(bits), codes, scales, workspace, s),
                    "rsq_layer_fused correction launch");
    if (st != RSQ_OK) return st;
    return hip_status(rsq::launch_qgemm(codes, scales, n, w_codes, w_scales, n_out, d, code_format(bits), y, y_dtype,
                                        n_out, nullptr, nullptr, 0, workspace, s),
                      "rsq_layer_fused GEMM launch");
}

}  // extern "C"
