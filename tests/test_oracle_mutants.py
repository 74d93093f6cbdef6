"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle function for a plausible wrong version (dropped
-I_r, transposed M, wrong sign, off-by-one rounding, wrong tie rule, swapped
nibbles) and re-runs the pin that should fail. If a pin passed with the
mutant in place, it would not be pinning that step.
"""
import numpy as np
import pytest

from oracle import online, packing, prep

import test_oracle_online as T_on
import test_oracle_prep as T_pre


def _expect_failure(fn):
    with pytest.raises(AssertionError):
        fn()


def test_dropped_identity_in_subspace_transform_is_caught(monkeypatch):
    monkeypatch.setattr(prep, "subspace_transform", lambda t, u: u.T @ t @ u)
    _expect_failure(T_on.test_global_rotation_site_is_identity)
    _expect_failure(T_on.test_rank_d_equals_dense_product)


def test_transposed_subspace_transform_is_caught(monkeypatch):
    monkeypatch.setattr(prep, "subspace_transform", lambda t, u: (u.T @ t @ u - np.eye(u.shape[1])).T)
    _expect_failure(T_on.test_rank_d_equals_dense_product)
    _expect_failure(T_on.test_two_dimensional_rotation_worked_case)


def test_wrong_mismatch_orientation_is_caught(monkeypatch):
    monkeypatch.setattr(prep, "basis_mismatch", lambda r_in, r_out: r_out @ r_in.T)
    _expect_failure(T_pre.test_mismatch_orientation)


def test_sign_error_in_reprojection_is_caught(monkeypatch):
    monkeypatch.setattr(online, "reproject", lambda h, c, u: np.asarray(h, np.float64) - c @ np.asarray(u, np.float64).T)
    _expect_failure(T_on.test_rank_d_equals_dense_product)
    _expect_failure(T_on.test_float32_operator_is_orthogonal_and_norm_preserving)


def test_right_instead_of_left_projection_is_caught(monkeypatch):
    monkeypatch.setattr(online, "project", lambda h, u: np.asarray(h, np.float64)[:, : u.shape[1]])
    _expect_failure(T_on.test_rank_d_equals_dense_product)


def test_cayley_sign_error_is_caught(monkeypatch):
    def bad(s):
        eye = np.eye(s.shape[0])
        return np.linalg.solve(eye + s, eye + s)
    monkeypatch.setattr(prep, "cayley", bad)
    _expect_failure(lambda: T_pre.test_cayley_two_by_two_closed_form(0.3))


def test_round_half_away_from_zero_is_caught(monkeypatch):
    def bad(a, bits):
        a = np.atleast_2d(np.asarray(a, np.float32))
        qm = np.float32(packing.qmax(bits))
        s = (np.max(np.abs(a), axis=1) / qm).astype(np.float32)
        q = np.sign(a) * np.floor(np.abs(a / s[:, None]) + 0.5)
        return np.clip(q, -qm, qm).astype(np.int64), s
    monkeypatch.setattr(online, "quantize", bad)
    _expect_failure(T_on.test_quantiser_worked_examples)
    _expect_failure(lambda: T_on.test_quantiser_matches_brute_force(4))


def test_scale_with_wrong_qmax_is_caught(monkeypatch):
    monkeypatch.setattr(online, "qmax", lambda bits: 1 << (bits - 1))
    _expect_failure(T_on.test_quantiser_worked_examples)


def test_swapped_nibbles_are_caught(monkeypatch):
    orig = packing.pack

    def bad(codes, bits):
        p = orig(codes, bits)
        return ((p >> 4) | (p << 4)).astype(np.uint8) if bits == 4 else p
    monkeypatch.setattr(packing, "pack", bad)
    _expect_failure(T_on.test_packing_hand_worked_bytes)


def test_rmsnorm_missing_eps_is_caught(monkeypatch):
    monkeypatch.setattr(online, "rms_inv", lambda x, eps: (1.0 / np.sqrt(np.mean(np.asarray(x, np.float64) ** 2, axis=-1))).astype(np.float32))
    _expect_failure(T_on.test_rmsnorm_mean_square_closed_form)


def test_dequant_missing_weight_scale_is_caught(monkeypatch):
    monkeypatch.setattr(online, "dequant", lambda acc, sa, sw, dt: (np.asarray(acc).astype(np.float32) * np.asarray(sa, np.float32)[:, None]))
    _expect_failure(T_on.test_dequant_equals_scaled_float64_sum)


def test_fp4_mistakes_are_caught(monkeypatch):
    real_pack, real_value = packing.pack_fp4, packing.e2m1_value
    # nibbles of a byte swapped
    monkeypatch.setattr(packing, "pack_fp4", lambda c: (lambda p: ((p << 4) | (p >> 4)).astype(np.uint8))(real_pack(c)))
    _expect_failure(T_on.test_fp4_packing_hand_worked_bytes)
    monkeypatch.setattr(packing, "pack_fp4", real_pack)
    # exponent bias 0 instead of 1 (every normal value doubled)
    monkeypatch.setattr(packing, "e2m1_value",
                        lambda n: real_value(n) * (2.0 if (n >> 1) & 3 else 1.0))
    _expect_failure(T_on.test_e2m1_values_match_the_mx_table)
    # codes stored as plain two's complement nibbles
    monkeypatch.setattr(packing, "e2m1_value", real_value)

    def twos(c):
        c = np.atleast_2d(np.asarray(c, np.int64))
        out = np.zeros((c.shape[0], c.shape[1] // 2), np.int64)
        for i in range(4):
            for b in range(4):
                out[:, 16 * np.arange(c.shape[1] // 32) + 4 * i + b] = ((c[:, 8 * i + b::32] & 15) << 4) | (c[:, 8 * i + 4 + b::32] & 15)
        return out.astype(np.uint8)
    monkeypatch.setattr(packing, "pack_fp4", twos)
    _expect_failure(T_on.test_fp4_packing_hand_worked_bytes)


def test_site_b_reading_the_uncorrected_residual_is_caught(monkeypatch):
    real = online.layer_linear_path

    def bad(h, site_a, site_b, weights, o_in, down_in, h_dtype, bits, eps, y_dtype):
        out = real(h, site_a, site_b, weights, o_in, down_in, h_dtype, bits, eps, y_dtype)
        b = online.layer_fused(h, *site_b, h_dtype, bits, eps, *weights["gate_up"], y_dtype)  # h, not site A's h'
        out["siteB"], out["gate_up"] = b, b["y"]
        return out
    monkeypatch.setattr(online, "layer_linear_path", bad)
    _expect_failure(T_on.test_layer_linear_path_wires_each_linear_to_its_input)


def test_linears_fed_the_wrong_inputs_are_caught(monkeypatch):
    real = online.layer_linear_path

    def bad(h, site_a, site_b, weights, o_in, down_in, h_dtype, bits, eps, y_dtype):
        out = real(h, site_a, site_b, weights, o_in, down_in, h_dtype, bits, eps, y_dtype)
        out["qkv"], out["gate_up"] = (online.qgemm_packed(out["siteB"]["codes"], out["siteB"]["scales"],
                                                          *weights["qkv"], out["siteB"]["q"].shape[1], bits, y_dtype)[0],
                                      out["gate_up"])
        return out
    monkeypatch.setattr(online, "layer_linear_path", bad)
    _expect_failure(T_on.test_layer_linear_path_wires_each_linear_to_its_input)


def test_quantising_the_uncorrected_residual_is_caught(monkeypatch):
    def bad(h, u, m, h_dtype, bits, eps, w_codes, w_scales, y_dtype, norm_weight=None):
        hp = online.correct(h, u, m, h_dtype)
        codes, scales, q = online.quant_act_packed(h, bits, True, eps, norm_weight)   # h instead of h'
        y, acc = online.qgemm_packed(codes, scales, w_codes, w_scales, np.asarray(h).shape[1], bits, y_dtype)
        return {"h_out": hp, "codes": codes, "scales": scales, "q": q, "y": y, "acc": acc}
    monkeypatch.setattr(online, "layer_fused", bad)
    _expect_failure(T_on.test_layer_fused_with_a_quarter_turn_site)
    _expect_failure(T_on.test_layer_linear_path_wires_each_linear_to_its_input)


def test_transposed_fusion_rotation_is_caught(monkeypatch):
    real = prep.fuse_weight
    monkeypatch.setattr(prep, "fuse_weight",
                        lambda w, right=None, left=None: real(w, None if right is None else np.asarray(right).T,
                                                              None if left is None else np.asarray(left).T))
    _expect_failure(T_pre.test_fused_linear_on_the_rotated_input_is_the_original_linear)
