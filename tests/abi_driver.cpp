// Host-only check of the C ABI's argument handling, built with the address
// and undefined-behaviour sanitizers (tests/test_abi_sanitized.py). The kernel
// launchers are replaced by recorders, so every case can assert whether the
// call reached a launch (nothing may be enqueued after a failed check) and
// how a launch failure is reported; no device is needed.
#include <cstdio>
#include <cstring>

#include "rsq.h"
#include "../rotation_bit_post_amd/csrc/rsq_internal.h"

namespace {
int g_launches = 0;
hipError_t g_ret = hipSuccess;
const void *g_res = nullptr;
int64_t g_ld_r = -1;
int g_bits = -1;
void *g_ws = nullptr;
bool g_left = false;
size_t g_need_c = 0, g_need_g = 0;
int g_fail = 0, g_cases = 0;

void expect(const char *what, int got, int want, int launches) {
    ++g_cases;
    const bool msg_ok = want == RSQ_OK || std::strlen(rsq_last_error()) > 0;
    if (got != want || g_launches != launches || !msg_ok) {
        std::printf("FAIL %s: status %d (want %d), launches %d (want %d), message '%s'\n", what, got, want, g_launches,
                    launches, rsq_last_error());
        ++g_fail;
    }
    g_launches = 0;
}
}  // namespace

namespace rsq {
int device_cus() { return 256; }
hipError_t launch_site_prepare(const float *, const float *, int, int, void *, hipStream_t) {
    ++g_launches;
    return g_ret;
}
hipError_t launch_correct(const void *, void *, int, int64_t, int, int64_t, const void *, int, bool, const float *,
                          float, int, uint8_t *, float *, void *ws, hipStream_t) {
    ++g_launches;
    g_ws = ws;
    return g_ret;
}
size_t correct_workspace_bytes(int64_t, int64_t) { return g_need_c; }
size_t qgemm_workspace_bytes(int64_t, int64_t, int64_t, int) { return g_need_g; }
hipError_t launch_quant(const void *, int, int64_t, int, int64_t, bool, const float *, float, int, uint8_t *, float *,
                        hipStream_t) {
    ++g_launches;
    return g_ret;
}
hipError_t launch_qgemm(const uint8_t *, const float *, int64_t, const uint8_t *, const float *, int64_t, int64_t,
                        int bits, void *, int, int64_t, int32_t *, const void *res, int64_t ld_r, void *ws,
                        hipStream_t) {
    ++g_launches;
    g_ws = ws;
    g_res = res;
    g_ld_r = ld_r;
    g_bits = bits;
    return g_ret;
}
hipError_t launch_codes_to_fp4(const uint8_t *, int64_t, int64_t, uint8_t *, hipStream_t) {
    ++g_launches;
    return g_ret;
}
hipError_t launch_rotate_weight(const float *, int64_t, int64_t, const float *, bool left, float *, hipStream_t) {
    ++g_launches;
    g_left = left;
    return g_ret;
}
}  // namespace rsq

int main() {
    alignas(16) static unsigned char mem[1 << 20];
    unsigned char *p = mem, *q = mem + (1 << 19);
    const float *f = reinterpret_cast<const float *>(mem);
    float *fo = reinterpret_cast<float *>(q);

    // queries
    expect("row bytes int4", rsq_packed_row_bytes(64, 4) == 32 ? 0 : 1, 0, 0);
    expect("row bytes int3", rsq_packed_row_bytes(64, 3) == 24 ? 0 : 1, 0, 0);
    expect("row bytes bad", rsq_packed_row_bytes(48, 4) == 0 ? 0 : 1, 0, 0);
    expect("site bytes", rsq_site_bytes(256, 8) == 256u * 32 * 8 ? 0 : 1, 0, 0);
    expect("site bytes r > 64", rsq_site_bytes(256, 65) == 0 ? 0 : 1, 0, 0);
    expect("status strings", std::strcmp(rsq_status_str(RSQ_ERR_HIP), "RSQ_ERR_HIP") == 0 ? 0 : 1, 0, 0);

    // site preparation
    expect("site ok", rsq_site_prepare(f, f, 256, 8, q, nullptr), RSQ_OK, 1);
    expect("site r = 0", rsq_site_prepare(f, f, 256, 0, q, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("site r > 64", rsq_site_prepare(f, f, 256, 65, q, nullptr), RSQ_ERR_UNSUPPORTED, 0);
    expect("site d % 32", rsq_site_prepare(f, f, 250, 8, q, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("site null", rsq_site_prepare(nullptr, f, 256, 8, q, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("site misaligned", rsq_site_prepare(f, f, 256, 8, q + 4, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("site d too wide", rsq_site_prepare(f, f, 32 * 512, 8, q, nullptr), RSQ_ERR_UNSUPPORTED, 0);

    // correction
    expect("correct ok", rsq_subspace_correct(p, q, RSQ_BF16, 4, 256, 256, p, 8, nullptr), RSQ_OK, 1);
    expect("correct in place", rsq_subspace_correct(p, p, RSQ_BF16, 4, 256, 256, q, 8, nullptr), RSQ_OK, 1);
    expect("correct n = 0", rsq_subspace_correct(nullptr, nullptr, RSQ_BF16, 0, 256, 256, nullptr, 8, nullptr), RSQ_OK, 0);
    expect("correct dtype", rsq_subspace_correct(p, q, 7, 4, 256, 256, p, 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct n < 0", rsq_subspace_correct(p, q, RSQ_BF16, -1, 256, 256, p, 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct ld < d", rsq_subspace_correct(p, q, RSQ_BF16, 4, 256, 128, p, 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct stride", rsq_subspace_correct(p, q, RSQ_BF16, 4, 256, 260, p, 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct overlap", rsq_subspace_correct(p, p + 16, RSQ_BF16, 4, 256, 256, q, 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct null", rsq_subspace_correct(p, q, RSQ_BF16, 4, 256, 256, nullptr, 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct f32 too wide", rsq_subspace_correct(p, q, RSQ_F32, 1, 8192, 8192, p, 8, nullptr), RSQ_ERR_UNSUPPORTED, 0);
    expect("correct bf16 widest", rsq_subspace_correct(p, p, RSQ_BF16, 1, 8192, 8192, q, 8, nullptr), RSQ_OK, 1);

    // quantisation
    expect("quant ok", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, RSQ_QA_RMSNORM, nullptr, 1e-5f, 4, q, fo, nullptr), RSQ_OK, 1);
    expect("quant bits", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, 0, nullptr, 0.0f, 5, q, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant flags", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, 2u, nullptr, 0.0f, 4, q, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant eps", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, RSQ_QA_RMSNORM, nullptr, -1.0f, 4, q, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant k", rsq_quant_act(p, RSQ_BF16, 4, 40, 40, 0, nullptr, 0.0f, 4, q, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant k max", rsq_quant_act(p, RSQ_BF16, 4, 32800, 32800, 0, nullptr, 0.0f, 4, q, fo, nullptr), RSQ_ERR_UNSUPPORTED, 0);
    expect("quant null x", rsq_quant_act(nullptr, RSQ_BF16, 4, 256, 256, 0, nullptr, 0.0f, 4, q, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant misaligned codes", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, 0, nullptr, 0.0f, 4, q + 2, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);

    // fused correction + quantisation, and one site with its linear
    expect("correct_quant ok", rsq_correct_quant(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 3, q + 4096, fo + 4096, nullptr, 0, nullptr), RSQ_OK, 1);
    expect("correct_quant eps", rsq_correct_quant(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, -1.0f, 3, q + 4096, fo + 4096, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("layer_fused ok", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, p, f, 64, q + 8192, RSQ_BF16, nullptr, 0, nullptr), RSQ_OK, 2);
    expect("layer_fused n_out", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, p, f, 48, q + 8192, RSQ_BF16, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);

    // GEMMs
    expect("qgemm ok", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 1);
    expect("qgemm n = 0", rsq_qgemm(nullptr, nullptr, 0, nullptr, nullptr, 64, 128, 4, nullptr, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 0);
    expect("qgemm bits", rsq_qgemm(p, f, 4, p, f, 64, 128, 2, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("qgemm n_out", rsq_qgemm(p, f, 4, p, f, 40, 128, 4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("qgemm k max", rsq_qgemm(p, f, 4, p, f, 64, 65568, 4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_UNSUPPORTED, 0);
    expect("qgemm ld_y", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 32, nullptr, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("qgemm acc misaligned", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, reinterpret_cast<int32_t *>(q + 4), nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("residual ok", rsq_qgemm_residual(p, f, 4, p, f, 64, 128, 4, q, 64, q + 65536, RSQ_BF16, 64, nullptr, 0, nullptr), RSQ_OK, 1);
    if (g_res != q || g_ld_r != 64) { std::printf("FAIL residual not passed to the launcher\n"); ++g_fail; }
    expect("residual in place", rsq_qgemm_residual(p, f, 4, p, f, 64, 128, 4, q, 64, q, RSQ_BF16, 64, nullptr, 0, nullptr), RSQ_OK, 1);
    expect("residual in place ld", rsq_qgemm_residual(p, f, 4, p, f, 64, 128, 4, q, 96, q, RSQ_BF16, 64, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("residual overlap", rsq_qgemm_residual(p, f, 4, p, f, 64, 128, 4, q, 64, q + 64, RSQ_BF16, 64, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("residual null", rsq_qgemm_residual(p, f, 4, p, f, 64, 128, 4, nullptr, 64, q, RSQ_BF16, 64, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);

    // fp4 codes: conversion and the linear on them
    expect("to_fp4 ok", rsq_codes_to_fp4(p, 4, 256, q, nullptr), RSQ_OK, 1);
    expect("to_fp4 rows = 0", rsq_codes_to_fp4(nullptr, 0, 256, nullptr, nullptr), RSQ_OK, 0);
    expect("to_fp4 k", rsq_codes_to_fp4(p, 4, 250, q, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("to_fp4 rows < 0", rsq_codes_to_fp4(p, -1, 256, q, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("to_fp4 overlap", rsq_codes_to_fp4(p, 4, 256, p + 256, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("to_fp4 misaligned", rsq_codes_to_fp4(p, 4, 256, q + 8, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("to_fp4 null", rsq_codes_to_fp4(p, 4, 256, nullptr, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("fp4 qgemm ok", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, nullptr, 0, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 1);
    if (g_bits != rsq::kFp4 || g_res != nullptr) { std::printf("FAIL fp4 qgemm: wrong code format or residual at the launcher\n"); ++g_fail; }
    expect("fp4 qgemm residual", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, q + 65536, 64, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 1);
    if (g_res != q + 65536 || g_ld_r != 64) { std::printf("FAIL fp4 qgemm: residual not passed to the launcher\n"); ++g_fail; }
    expect("fp4 qgemm in place", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, q, 64, q, RSQ_F32, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 1);
    expect("fp4 qgemm in place ld", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, q, 96, q, RSQ_F32, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("fp4 qgemm overlap", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, q + 64, 64, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("fp4 qgemm k max", rsq_qgemm_fp4(p, f, 4, p, f, 64, 65568, nullptr, 0, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_UNSUPPORTED, 0);
    expect("fp4 qgemm n = 0", rsq_qgemm_fp4(nullptr, nullptr, 0, nullptr, nullptr, 64, 128, nullptr, 0, nullptr, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 0);
    expect("fp4 qgemm acc misaligned", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, nullptr, 0, q, RSQ_BF16, 64, reinterpret_cast<int32_t *>(q + 4), nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("qgemm int3 format", rsq_qgemm(p, f, 4, p, f, 64, 128, 3, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 1);
    if (g_bits != 3) { std::printf("FAIL int3 qgemm: wrong code format at the launcher\n"); ++g_fail; }
    expect("qgemm fp4 bits", rsq_qgemm(p, f, 4, p, f, 64, 128, 3 | RSQ_FP4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_OK, 1);
    if (g_bits != rsq::kFp4) { std::printf("FAIL qgemm bits 3 | RSQ_FP4: wrong code format at the launcher\n"); ++g_fail; }
    expect("qgemm 4 | RSQ_FP4", rsq_qgemm(p, f, 4, p, f, 64, 128, 4 | RSQ_FP4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant fp4 codes", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, RSQ_QA_RMSNORM, nullptr, 1e-5f, 3 | RSQ_FP4, q, fo, nullptr), RSQ_OK, 1);
    expect("correct_quant fp4 codes", rsq_correct_quant(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 3 | RSQ_FP4, q + 4096, fo + 4096, nullptr, 0, nullptr), RSQ_OK, 1);
    expect("layer_fused fp4", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 3 | RSQ_FP4, q + 4096, fo + 4096, p, f, 64, q + 8192, RSQ_BF16, nullptr, 0, nullptr), RSQ_OK, 2);
    if (g_bits != rsq::kFp4) { std::printf("FAIL layer_fused bits 3 | RSQ_FP4: wrong code format at the GEMM\n"); ++g_fail; }
    expect("row bytes fp4", rsq_packed_row_bytes(64, 3 | RSQ_FP4) == 32 ? 0 : 1, 0, 0);

    // workspace: sized by the queries, checked before any launch, passed to the launchers
    g_need_g = 4096;
    expect("query qgemm ws", rsq_qgemm_workspace_bytes(4, 64, 128, 4) == 4096 ? 0 : 1, 0, 0);
    expect("query qgemm ws bad k", rsq_qgemm_workspace_bytes(4, 64, 100, 4) == 0 ? 0 : 1, 0, 0);
    expect("query qgemm ws bad bits", rsq_qgemm_workspace_bytes(4, 64, 128, 5) == 0 ? 0 : 1, 0, 0);
    expect("qgemm ws missing", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_WORKSPACE, 0);
    expect("qgemm ws small", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, nullptr, q + 65536, 4095, nullptr), RSQ_ERR_WORKSPACE, 0);
    expect("qgemm ws misaligned", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, nullptr, q + 65540, 8192, nullptr), RSQ_ERR_WORKSPACE, 0);
    expect("qgemm ws ok", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, nullptr, q + 65536, 4096, nullptr), RSQ_OK, 1);
    if (g_ws != q + 65536) { std::printf("FAIL qgemm: workspace not passed to the launcher\n"); ++g_fail; }
    expect("residual ws missing", rsq_qgemm_residual(p, f, 4, p, f, 64, 128, 4, q, 64, q, RSQ_BF16, 64, nullptr, 0, nullptr), RSQ_ERR_WORKSPACE, 0);
    expect("fp4 qgemm ws missing", rsq_qgemm_fp4(p, f, 4, p, f, 64, 128, nullptr, 0, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_WORKSPACE, 0);
    g_need_g = 0;
    g_need_c = 1024;
    expect("query correct ws", rsq_correct_workspace_bytes(4, 256) == 1024 ? 0 : 1, 0, 0);
    expect("query correct ws bad d", rsq_correct_workspace_bytes(4, 250) == 0 ? 0 : 1, 0, 0);
    expect("correct_quant ws missing", rsq_correct_quant(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, nullptr, 0, nullptr), RSQ_ERR_WORKSPACE, 0);
    expect("correct_quant ws ok", rsq_correct_quant(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, q + 65536, 1024, nullptr), RSQ_OK, 1);
    if (g_ws != q + 65536) { std::printf("FAIL correct_quant: workspace not passed to the launcher\n"); ++g_fail; }
    expect("correction alone needs none", rsq_subspace_correct(p, q, RSQ_BF16, 4, 256, 256, p, 8, nullptr), RSQ_OK, 1);
    g_need_g = 2048;
    expect("query layer ws", rsq_layer_workspace_bytes(4, 256, 64, 4) == 2048 ? 0 : 1, 0, 0);
    expect("layer_fused ws small", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, p, f, 64, q + 8192, RSQ_BF16, q + 65536, 1024, nullptr), RSQ_ERR_WORKSPACE, 0);
    expect("layer_fused ws ok", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, p, f, 64, q + 8192, RSQ_BF16, q + 65536, 2048, nullptr), RSQ_OK, 2);
    g_need_c = g_need_g = 0;
    // norm weights are read with 16-byte loads
    expect("quant norm_w misaligned", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, RSQ_QA_RMSNORM, f + 1, 1e-5f, 4, q, fo, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("correct_quant norm_w misaligned", rsq_correct_quant(p, q, RSQ_BF16, 4, 256, p, 8, f + 2, 1e-5f, 4, q + 4096, fo + 4096, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("layer_fused norm_w misaligned", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, f + 3, 1e-5f, 4, q + 4096, fo + 4096, p, f, 64, q + 8192, RSQ_BF16, nullptr, 0, nullptr), RSQ_ERR_INVALID_ARG, 0);
    expect("quant norm_w aligned", rsq_quant_act(p, RSQ_BF16, 4, 256, 256, RSQ_QA_RMSNORM, f + 4, 1e-5f, 4, q, fo, nullptr), RSQ_OK, 1);

    // offline weight fusion
    {
        const float *wf = reinterpret_cast<const float *>(p);
        float *wo = reinterpret_cast<float *>(q);
        const float *rf = reinterpret_cast<const float *>(q + 65536);
        expect("rotate right", rsq_rotate_weight(wf, 64, 96, rf, RSQ_ROTATE_RIGHT, wo, nullptr), RSQ_OK, 1);
        if (g_left) { std::printf("FAIL rotate right reached the launcher as left\n"); ++g_fail; }
        expect("rotate left", rsq_rotate_weight(wf, 64, 96, rf, RSQ_ROTATE_LEFT, wo, nullptr), RSQ_OK, 1);
        if (!g_left) { std::printf("FAIL rotate left reached the launcher as right\n"); ++g_fail; }
        expect("rotate side", rsq_rotate_weight(wf, 64, 96, rf, 2, wo, nullptr), RSQ_ERR_INVALID_ARG, 0);
        expect("rotate k", rsq_rotate_weight(wf, 64, 100, rf, RSQ_ROTATE_RIGHT, wo, nullptr), RSQ_ERR_INVALID_ARG, 0);
        expect("rotate null", rsq_rotate_weight(wf, 64, 96, nullptr, RSQ_ROTATE_RIGHT, wo, nullptr), RSQ_ERR_INVALID_ARG, 0);
        expect("rotate in place", rsq_rotate_weight(wf, 64, 96, rf, RSQ_ROTATE_RIGHT, const_cast<float *>(wf), nullptr), RSQ_ERR_INVALID_ARG, 0);
        expect("rotate overlaps R", rsq_rotate_weight(wf, 64, 96, rf, RSQ_ROTATE_RIGHT, wo + 16384, nullptr), RSQ_ERR_INVALID_ARG, 0);
        expect("rotate misaligned", rsq_rotate_weight(wf + 1, 64, 96, rf, RSQ_ROTATE_RIGHT, wo, nullptr), RSQ_ERR_INVALID_ARG, 0);
        expect("rotate too large", rsq_rotate_weight(wf, 64, (1 << 20) + 32, rf, RSQ_ROTATE_RIGHT, wo, nullptr), RSQ_ERR_UNSUPPORTED, 0);
    }

    // a launch failure surfaces as RSQ_ERR_HIP with a message; the fused call stops after the failed launch
    g_ret = hipErrorInvalidValue;
    expect("launch failure", rsq_qgemm(p, f, 4, p, f, 64, 128, 4, q, RSQ_BF16, 64, nullptr, nullptr, 0, nullptr), RSQ_ERR_HIP, 1);
    expect("launch failure to_fp4", rsq_codes_to_fp4(p, 4, 256, q, nullptr), RSQ_ERR_HIP, 1);
    expect("launch failure fused", rsq_layer_fused(p, q, RSQ_BF16, 4, 256, p, 8, nullptr, 1e-5f, 4, q + 4096, fo + 4096, p, f, 64, q + 8192, RSQ_BF16, nullptr, 0, nullptr), RSQ_ERR_HIP, 1);
    g_ret = hipSuccess;

    std::printf("%s: %d cases, %d failed\n", g_fail ? "FAILED" : "ok", g_cases, g_fail);
    return g_fail != 0;
}
