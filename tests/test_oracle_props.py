"""Randomised properties of the oracle (CPU only, hypothesis).

Each property follows from the mathematics of the step, not from its code:
the correction is linear in h, is the identity for M = 0, equals the dense
h T when the basis spans the whole space (r = D), and preserves the norm when
the basis is a T-invariant subspace (the top singular subspace of T - I for
an orthogonal T); the quantiser's codes stay in range, reconstruct every
element to within half a step, map the largest magnitude to +-qmax and scale
with the input; packing round-trips; the integer GEMM equals plain integer
loops. Shapes are drawn small (D a multiple of 32, token counts with tails).
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import assume, given, settings, strategies as st  # noqa: E402

from oracle import online, packing, prep  # noqa: E402

SETTINGS = settings(max_examples=25, deadline=None, derandomize=True)


def _skew(d, rng):
    g = rng.standard_normal((d, d))
    u = np.triu(g, 1)
    return u - u.T


def _orthonormal(d, r, rng):
    q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return q


@SETTINGS
@given(d=st.sampled_from([32, 64, 96, 128]), r=st.integers(1, 16), n=st.integers(1, 17), seed=st.integers(0, 2**31))
def test_correction_is_linear_in_h(d, r, n, seed):
    rng = np.random.default_rng(seed)
    u = _orthonormal(d, min(r, d), rng)
    m = rng.standard_normal((u.shape[1], u.shape[1]))
    h1, h2 = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    a, b = rng.standard_normal(2)

    def f(h):
        return online.reproject(h, online.transform(online.project(h, u), m), u)

    lhs = f(a * h1 + b * h2)
    rhs = a * f(h1) + b * f(h2)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12 * np.abs(rhs).max())


@SETTINGS
@given(d=st.sampled_from([32, 64, 128]), r=st.integers(1, 32), n=st.integers(1, 17),
       dtype=st.sampled_from(["f32", "bf16"]), seed=st.integers(0, 2**31))
def test_zero_transform_leaves_stored_rows_unchanged(d, r, n, dtype, seed):
    rng = np.random.default_rng(seed)
    u = _orthonormal(d, min(r, d), rng)
    h = online.correct(rng.standard_normal((n, d)) * 7, np.eye(d)[:, :1], np.zeros((1, 1)), dtype)  # storage values
    out = online.correct(h, u, np.zeros((u.shape[1], u.shape[1])), dtype)
    assert np.array_equal(np.asarray(out, np.float64), np.asarray(h, np.float64))


@SETTINGS
@given(d=st.sampled_from([32, 64]), n=st.integers(1, 9), seed=st.integers(0, 2**31))
def test_full_rank_basis_gives_the_dense_product(d, n, seed):
    rng = np.random.default_rng(seed)
    t = prep.basis_mismatch(prep.rotation(_skew(d, rng), 0.05), prep.rotation(_skew(d, rng), 0.05))
    u = _orthonormal(d, d, rng)          # any orthonormal basis of the whole space
    m = prep.subspace_transform(t, u)
    h = rng.standard_normal((n, d))
    out = online.reproject(h, online.transform(online.project(h, u), m), u)
    assert np.allclose(out, h @ t, rtol=0, atol=1e-11 * np.abs(h).max())


@SETTINGS
@given(d=st.sampled_from([32, 64, 128]), half_r=st.integers(1, 8), n=st.integers(1, 9), seed=st.integers(0, 2**31))
def test_invariant_subspace_correction_preserves_the_norm(d, half_r, n, seed):
    rng = np.random.default_rng(seed)
    r = 2 * half_r
    a_in, a_out = _skew(d, rng), _skew(d, rng)
    try:
        s = prep.site(a_in, a_out, 0.05, r)
    except ValueError:          # no singular-value gap at this rank: the subspace is not defined
        assume(False)
        return
    h = rng.standard_normal((n, d))
    out = online.reproject(h, online.transform(online.project(h, s["U"]), s["M"]), s["U"])
    assert np.allclose(np.linalg.norm(out, axis=1), np.linalg.norm(h, axis=1), rtol=1e-9)


@SETTINGS
@given(k=st.sampled_from([32, 64, 96, 160]), n=st.integers(1, 17), bits=st.sampled_from([3, 4]),
       scale=st.floats(1e-3, 1e3), seed=st.integers(0, 2**31))
def test_quantiser_bounds_extremes_and_reconstruction(k, n, bits, scale, seed):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((n, k)) * scale).astype(np.float32)
    q, s = online.quantize(a, bits)
    qm = packing.qmax(bits)
    assert q.min() >= -qm and q.max() <= qm
    assert np.all(s > 0)
    # the element of largest magnitude of each row lands on +-qmax
    idx = np.argmax(np.abs(a), axis=1)
    assert np.array_equal(np.abs(q[np.arange(n), idx]), np.full(n, qm))
    # every element is reconstructed to within half a step (float32 quotient slack)
    err = np.abs(a.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6) + 1e-30)


@SETTINGS
@given(k=st.sampled_from([32, 64]), n=st.integers(1, 9), bits=st.sampled_from([3, 4]),
       e=st.integers(-20, 20), seed=st.integers(0, 2**31))
def test_quantiser_commutes_with_power_of_two_scaling(k, n, bits, e, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, k)).astype(np.float32)
    q1, s1 = online.quantize(a, bits)
    q2, s2 = online.quantize(a * np.float32(2.0 ** e), bits)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(2.0 ** e))


@SETTINGS
@given(k32=st.integers(1, 6), n=st.integers(1, 9), bits=st.sampled_from([3, 4]), seed=st.integers(0, 2**31))
def test_pack_round_trip_and_row_bytes(k32, n, bits, seed):
    k = 32 * k32
    rng = np.random.default_rng(seed)
    qm = packing.qmax(bits)
    q = rng.integers(-qm, qm + 1, (n, k))
    packed = packing.pack(q, bits)
    assert packed.shape == (n, k * bits // 8) == (n, packing.packed_row_bytes(k, bits))
    assert np.array_equal(packing.unpack(packed, k, bits), q)


@SETTINGS
@given(n=st.integers(1, 5), nn=st.integers(1, 5), k=st.integers(1, 40), bits=st.sampled_from([3, 4]),
       seed=st.integers(0, 2**31))
def test_integer_gemm_equals_plain_loops(n, nn, k, bits, seed):
    rng = np.random.default_rng(seed)
    qm = packing.qmax(bits)
    qa = rng.integers(-qm, qm + 1, (n, k))
    qw = rng.integers(-qm, qm + 1, (nn, k))
    ref = [[sum(int(qa[t, i]) * int(qw[j, i]) for i in range(k)) for j in range(nn)] for t in range(n)]
    assert np.array_equal(online.gemm(qa, qw), np.array(ref, np.int64))
