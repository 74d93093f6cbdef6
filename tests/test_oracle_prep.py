"""Pins of the oracle's offline steps (CPU only).

Each test checks a fact fixed by the pages or by the mathematics, not a
re-typing of the oracle's formula: orthogonality, closed forms of small
cases, the T = I special case of a global rotation, invariances.
"""
import numpy as np
import pytest

from oracle import prep


def _skew(d, seed):
    g = np.random.default_rng(seed).standard_normal((d, d))
    u = np.triu(g, 1)
    return u - u.T


@pytest.mark.parametrize("d", [1, 2, 4, 64, 256])
def test_hadamard_orthonormal(d):
    h = prep.hadamard(d)
    assert np.allclose(h @ h.T, np.eye(d), atol=1e-12)
    assert np.allclose(np.abs(h), 1 / np.sqrt(d), atol=1e-15)


def test_hadamard_order_two_by_hand():
    assert np.allclose(prep.hadamard(2), np.array([[1, 1], [1, -1]]) / np.sqrt(2), atol=1e-16)


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        prep.hadamard(12)


@pytest.mark.parametrize("a", [0.0, 0.3, -1.7])
def test_cayley_two_by_two_closed_form(a):
    # S = [[0, a], [-a, 0]]  ->  C = [[1 - a^2, 2a], [-2a, 1 - a^2]] / (1 + a^2)
    s = np.array([[0.0, a], [-a, 0.0]])
    expect = np.array([[1 - a * a, 2 * a], [-2 * a, 1 - a * a]]) / (1 + a * a)
    assert np.allclose(prep.cayley(s), expect, atol=1e-14)


@pytest.mark.parametrize("d,eps", [(16, 0.5), (64, 0.02), (256, 0.01)])
def test_cayley_orthogonal_det_plus_one(d, eps):
    c = prep.cayley(eps * _skew(d, d))
    assert np.allclose(c.T @ c, np.eye(d), atol=1e-12)
    assert np.isclose(np.linalg.det(c), 1.0, atol=1e-9)


def test_global_rotation_gives_identity_mismatch():
    # A single rotation shared by input and output: T = I (it §2B, nl §2B).
    r = prep.rotation(_skew(64, 1), 0.02)
    assert np.allclose(prep.basis_mismatch(r, r), np.eye(64), atol=1e-12)


def test_hadamard_cancels_in_mismatch():
    d = 128
    a_in, a_out = _skew(d, 2), _skew(d, 3)
    t = prep.basis_mismatch(prep.rotation(a_in, 0.01), prep.rotation(a_out, 0.01))
    t_direct = prep.cayley(0.01 * a_out).T @ prep.cayley(0.01 * a_in)
    assert np.allclose(t, t_direct, atol=1e-12)
    assert np.allclose(t.T @ t, np.eye(d), atol=1e-12)


def test_mismatch_orientation():
    # T maps the input basis to the output one: R_out T = R_in.
    d = 32
    r_in, r_out = prep.rotation(_skew(d, 4), 0.1), prep.rotation(_skew(d, 5), 0.1)
    assert np.allclose(r_out @ prep.basis_mismatch(r_in, r_out), r_in, atol=1e-12)


def test_singular_values_come_in_pairs():
    # dT of an orthogonal T is normal; each 2-D rotation plane gives a pair 2|sin(theta/2)|.
    d = 64
    t = prep.basis_mismatch(prep.rotation(_skew(d, 6), 0.05), prep.rotation(_skew(d, 7), 0.05))
    s = np.linalg.svd(t - np.eye(d), compute_uv=False)
    assert np.allclose(s[0::2], s[1::2], atol=1e-12)
    theta = np.abs(np.angle(np.linalg.eigvals(t)))
    assert np.allclose(np.sort(2 * np.sin(theta / 2))[::-1], s, atol=1e-10)


@pytest.mark.parametrize("r", [2, 8, 16])
def test_subspace_is_invariant_and_q_r_orthogonal(r):
    d = 64
    t = prep.basis_mismatch(prep.rotation(_skew(d, 8), 0.05), prep.rotation(_skew(d, 9), 0.05))
    u, _ = prep.principal_subspace(t, r)
    assert np.allclose(u.T @ u, np.eye(r), atol=1e-12)
    resid = (np.eye(d) - u @ u.T) @ t @ u
    assert np.max(np.abs(resid)) < 1e-10
    q = u.T @ t @ u
    assert np.allclose(q.T @ q, np.eye(r), atol=1e-10)
    t_hat = prep.approx_operator(u, prep.subspace_transform(t, u))
    assert np.allclose(t_hat.T @ t_hat, np.eye(d), atol=1e-10)


def test_odd_rank_rejected_by_gap_check():
    d = 32
    t = prep.basis_mismatch(prep.rotation(_skew(d, 10), 0.05), prep.rotation(_skew(d, 11), 0.05))
    with pytest.raises(ValueError):
        prep.principal_subspace(t, 7)


def test_rank_d_reproduces_dense_mismatch():
    d = 32
    t = prep.basis_mismatch(prep.rotation(_skew(d, 12), 0.05), prep.rotation(_skew(d, 13), 0.05))
    u, _ = prep.principal_subspace(t, d)
    assert np.allclose(prep.approx_operator(u, prep.subspace_transform(t, u)), t, atol=1e-12)


@pytest.mark.parametrize("r", [2, 4, 8, 16, 32])
def test_frobenius_error_closed_form(r):
    # ||T - T_hat_r||_F^2 equals the sum of the discarded squared singular values.
    d = 64
    t = prep.basis_mismatch(prep.rotation(_skew(d, 14), 0.05), prep.rotation(_skew(d, 15), 0.05))
    u, s = prep.principal_subspace(t, r)
    err = np.linalg.norm(t - prep.approx_operator(u, prep.subspace_transform(t, u))) ** 2
    assert np.isclose(err, np.sum(s[r:] ** 2), rtol=1e-9, atol=1e-13)


def test_operator_independent_of_basis_choice_inside_subspace():
    d, r = 64, 8
    t = prep.basis_mismatch(prep.rotation(_skew(d, 16), 0.05), prep.rotation(_skew(d, 17), 0.05))
    u, _ = prep.principal_subspace(t, r)
    w, _ = np.linalg.qr(np.random.default_rng(0).standard_normal((r, r)))
    op1 = prep.approx_operator(u, prep.subspace_transform(t, u))
    u2 = u @ w
    op2 = prep.approx_operator(u2, prep.subspace_transform(t, u2))
    assert np.allclose(op1, op2, atol=1e-12)


def test_site_rounds_inputs_to_float32():
    d, r = 64, 8
    s = prep.site(_skew(d, 18), _skew(d, 19), 0.05, r)
    assert s["U32"].dtype == np.float32 and s["M32"].dtype == np.float32
    assert s["U32"].shape == (d, r) and s["M32"].shape == (r, r)
    assert np.allclose(s["U32"], s["U"], atol=1e-7)


def test_weight_quantisation_is_per_output_channel():
    w = np.array([[0.1, -0.7, 0.35], [2.0, 1.0, -0.5]], np.float32)
    q, s = prep.quantize_weight(w, 4)
    assert np.allclose(s, np.array([0.7, 2.0], np.float32) / np.float32(7))
    assert q[0, 1] == -7 and q[1, 0] == 7


# ---------------------------------------------------------- weight fusion
def _orth(d, seed):
    return prep.rotation(_skew(d, seed), 0.05) if d & (d - 1) == 0 else prep.cayley(0.05 * _skew(d, seed))


def test_fused_linear_on_the_rotated_input_is_the_original_linear():
    # zh 2.2 / fr 2A: with h~ = h R, y = h W^T = h~ (W R)^T
    rng = np.random.default_rng(70)
    n, k = 5, 64
    w = (rng.standard_normal((48, k)) * 0.02).astype(np.float32)
    r = _orth(k, 71).astype(np.float32)
    h = rng.standard_normal((n, k))
    wt = prep.fuse_weight(w, right=r)
    y = h @ w.astype(np.float64).T
    y_fused = (h @ r.astype(np.float64)) @ wt.astype(np.float64).T
    assert np.max(np.abs(y_fused - y)) <= 1e-5 * np.max(np.abs(y))
    # an output basis R': y R' = h~ (R'^T W R)^T
    r_out = _orth(48, 72).astype(np.float32)
    wt2 = prep.fuse_weight(w, right=r, left=r_out)
    y_out = (h @ r.astype(np.float64)) @ wt2.astype(np.float64).T
    assert np.max(np.abs(y_out - y @ r_out.astype(np.float64))) <= 1e-5 * np.max(np.abs(y))


def test_fusion_closed_forms():
    rng = np.random.default_rng(73)
    w = rng.standard_normal((32, 64)).astype(np.float32)
    # identity rotations: the weight itself, bit for bit
    assert np.array_equal(prep.fuse_weight(w, right=np.eye(64, dtype=np.float32)), w)
    assert np.array_equal(prep.fuse_weight(w), w)
    # a permutation on the right permutes the columns; on the left it permutes the rows
    perm = rng.permutation(64)
    p = np.eye(64, dtype=np.float32)[:, perm]
    assert np.array_equal(prep.fuse_weight(w, right=p), w[:, perm])
    q = np.eye(32, dtype=np.float32)[:, rng.permutation(32)]
    assert np.array_equal(prep.fuse_weight(w, left=q), (q.T @ w).astype(np.float32))
    # H is symmetric and orthogonal: fusing it twice gives the weight back
    h = prep.hadamard(64).astype(np.float32)
    twice = prep.fuse_weight(prep.fuse_weight(w, right=h), right=h)
    assert np.max(np.abs(twice - w)) <= 1e-5 * np.max(np.abs(w))
    # an orthogonal fusion keeps the Frobenius norm
    wt = prep.fuse_weight(w, right=_orth(64, 74), left=_orth(32, 75))
    assert abs(np.linalg.norm(wt.astype(np.float64)) / np.linalg.norm(w.astype(np.float64)) - 1) < 1e-6
