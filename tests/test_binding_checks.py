"""The Python binding's argument checks (CPU only): a tensor that does not
match what a call is told (dtype, shape, row or column stride, size of a code
or scale buffer, residency) raises ValueError before the C call, so no kernel
can read or write past a buffer. CPU tensors are used throughout; the last
check of every call is that its tensors live on the GPU, so a well-formed CPU
call stops there."""
import pytest
import torch

import rotation_bit_post_amd as rsq

BF16, F32, U8 = torch.bfloat16, torch.float32, torch.uint8


def _site(d, r):
    return torch.zeros(rsq.rsq_site_bytes(d, r), dtype=U8)


def _raises(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_correction_outputs_must_match_the_input_layout():
    d, r, n = 256, 8, 4
    h = torch.zeros((n, d), dtype=BF16)
    site = _site(d, r)
    _raises("dtype", rsq.rsq_subspace_correct, h, torch.zeros((n, d), dtype=F32), site, r)
    _raises("dtype", rsq.rsq_subspace_correct, h.float(), torch.zeros((n, d), dtype=BF16), site, r)
    _raises("shape", rsq.rsq_subspace_correct, h, torch.zeros((n + 1, d), dtype=BF16), site, r)
    _raises("strides", rsq.rsq_subspace_correct, h, torch.zeros((n, d + 64), dtype=BF16)[:, :d], site, r)
    _raises("unit column stride", rsq.rsq_subspace_correct, h.t(), torch.zeros((d, n), dtype=BF16), site, r)
    _raises("site", rsq.rsq_subspace_correct, h, torch.zeros_like(h), _site(d, r)[:-16], r)
    _raises("device tensor", rsq.rsq_subspace_correct, h, torch.zeros_like(h), site, r)


def test_fused_entry_points_take_contiguous_rows_only():
    d, r, n, bits = 256, 8, 4, 4
    big = torch.zeros((n, d + 64), dtype=BF16)
    codes, scales = torch.zeros((n, d // 2), dtype=U8), torch.zeros(n, dtype=F32)
    _raises("contiguous", rsq.rsq_correct_quant, big[:, :d], big[:, :d], _site(d, r), r, codes, scales, bits)
    h = torch.zeros((n, d), dtype=BF16)
    _raises("codes", rsq.rsq_correct_quant, h, torch.zeros_like(h), _site(d, r), r, codes[:-1], scales, bits)
    _raises("float32", rsq.rsq_correct_quant, h, torch.zeros_like(h), _site(d, r), r, codes, scales.double(), bits)
    _raises("norm_w", rsq.rsq_correct_quant, h, torch.zeros_like(h), _site(d, r), r, codes, scales, bits,
            norm_w=torch.ones(d - 32))
    _raises("workspace", rsq.rsq_correct_quant, h, torch.zeros_like(h), _site(d, r), r, codes, scales, bits,
            workspace=torch.zeros(64, dtype=torch.int32))
    _raises("device tensor", rsq.rsq_correct_quant, h, torch.zeros_like(h), _site(d, r), r, codes, scales, bits)
    w_codes, w_scales = torch.zeros((64, d // 2), dtype=U8), torch.zeros(64, dtype=F32)
    y = torch.zeros((n, 64), dtype=BF16)
    _raises("y must be contiguous", rsq.rsq_layer_fused, h, torch.zeros_like(h), _site(d, r), r, codes, scales,
            w_codes, w_scales, 64, torch.zeros((n, 128), dtype=BF16)[:, :64], bits)
    _raises("w_codes", rsq.rsq_layer_fused, h, torch.zeros_like(h), _site(d, r), r, codes, scales, w_codes[:32],
            w_scales, 64, y, bits)
    _raises("device tensor", rsq.rsq_layer_fused, h, torch.zeros_like(h), _site(d, r), r, codes, scales, w_codes,
            w_scales, 64, y, bits)


def test_quantiser_buffers_are_sized_from_the_packed_layout():
    n, k = 5, 224
    x = torch.zeros((n, k), dtype=BF16)
    _raises("codes", rsq.rsq_quant_act, x, torch.zeros((n, rsq.rsq_packed_row_bytes(k, 3) - 1), dtype=U8),
            torch.zeros(n, dtype=F32), 3)
    _raises("scales", rsq.rsq_quant_act, x, torch.zeros((n, k // 2), dtype=U8), torch.zeros(n - 1, dtype=F32), 4)
    _raises("no packed layout", rsq.rsq_quant_act, torch.zeros((n, 100), dtype=BF16), torch.zeros((n, 50), dtype=U8),
            torch.zeros(n, dtype=F32), 4)
    _raises("device tensor", rsq.rsq_quant_act, x, torch.zeros((n, k // 2), dtype=U8), torch.zeros(n, dtype=F32), 4)


def test_gemm_operands_and_outputs_are_checked():
    n, N, K, bits = 3, 64, 256, 4
    a, sa = torch.zeros((n, K // 2), dtype=U8), torch.zeros(n, dtype=F32)
    w, sw = torch.zeros((N, K // 2), dtype=U8), torch.zeros(N, dtype=F32)
    y = torch.zeros((n, N), dtype=BF16)
    _raises("a_codes", rsq.rsq_qgemm, a[:2], sa, n, w, sw, N, K, bits, y)
    _raises("w_scales", rsq.rsq_qgemm, a, sa, n, w, sw[:N - 1], N, K, bits, y)
    _raises("cannot hold", rsq.rsq_qgemm, a, sa, n, w, sw, N, K, bits, torch.zeros((n, N - 32), dtype=BF16))
    _raises("acc_out", rsq.rsq_qgemm, a, sa, n, w, sw, N, K, bits, y, acc_out=torch.zeros((n, N - 1), dtype=torch.int32))
    _raises("same dtype", rsq.rsq_qgemm_residual, a, sa, n, w, sw, N, K, bits, torch.zeros((n, N), dtype=F32), y)
    _raises("residual", rsq.rsq_qgemm_residual, a, sa, n, w, sw, N, K, bits, torch.zeros((n - 1, N), dtype=BF16), y)
    fa, fw = torch.zeros((n, K // 2), dtype=U8), torch.zeros((N, K // 2), dtype=U8)
    _raises("a_codes", rsq.rsq_qgemm_fp4, fa[:, :K // 4].contiguous(), sa, n, fw, sw, N, K, y)
    _raises("fp4", rsq.rsq_codes_to_fp4, torch.zeros((n, 3 * K // 8), dtype=U8), n, K, torch.zeros((n, K // 4), dtype=U8))
    _raises("device tensor", rsq.rsq_qgemm, a, sa, n, w, sw, N, K, bits, y)


def test_workspace_queries():
    # invalid sizes report no workspace; the call itself then reports the size
    assert rsq.rsq_qgemm_workspace_bytes(4, 100, 4096, 4) == 0
    assert rsq.rsq_qgemm_workspace_bytes(4, 128, 4000, 4) == 0
    assert rsq.rsq_qgemm_workspace_bytes(4, 128, 4096, 5) == 0
    assert rsq.rsq_correct_workspace_bytes(0, 4096) == 0
    assert rsq.rsq_correct_workspace_bytes(4, 100) == 0
    # no kernel of this version exchanges data between workgroups
    assert rsq.rsq_correct_workspace_bytes(1, 4096) == 0
    assert rsq.rsq_qgemm_workspace_bytes(64, 4096, 11008, 4) == 0
    for n in (1, 8, 64, 2048):
        for n_out, k in ((4096, 4096), (22016, 4096), (4096, 11008)):
            lw = rsq.rsq_layer_workspace_bytes(n, k, n_out, 4)
            assert lw == max(rsq.rsq_correct_workspace_bytes(n, k), rsq.rsq_qgemm_workspace_bytes(n, n_out, k, 4))
