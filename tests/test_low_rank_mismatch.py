"""The rank sweep's low-rank mismatch (CPU only).

Rotations H C(eps A) whose skew generators A have rank 2k differ from their
Hadamard start only inside a 2k-dimensional subspace, so T - I has rank at
most 4k. Then the method's premise holds exactly: the rank-4k subspace
correction reproduces the dense T, and lower ranks leave an error that falls
with r. These tests pin the generator and the oracle's behaviour on it.
"""
import numpy as np
import pytest

import synth
from oracle import online, prep

TINY = synth.WORKLOADS[synth.TINY]          # D = 256


@pytest.mark.parametrize("k", [1, 2, 4])
def test_low_rank_skew_is_skew_of_rank_2k_and_seeded(k):
    a = synth.low_rank_skew(TINY, "A", "in", k)
    assert a.shape == (TINY.D, TINY.D) and a.dtype == np.float64
    assert np.array_equal(a, -a.T)
    s = np.linalg.svd(a, compute_uv=False)
    assert np.sum(s > 1e-9 * s[0]) == 2 * k
    assert 0.2 < s[0] < 5.0                                   # spectral norm about 1
    assert np.array_equal(a, synth.low_rank_skew(TINY, "A", "in", k))
    assert not np.allclose(a, synth.low_rank_skew(TINY, "A", "out", k))
    with pytest.raises(ValueError):
        synth.low_rank_skew(TINY, "A", "in", TINY.D)


def _mismatch(k, eps):
    return prep.basis_mismatch(prep.rotation(synth.low_rank_skew(TINY, "A", "in", k), eps),
                               prep.rotation(synth.low_rank_skew(TINY, "A", "out", k), eps))


@pytest.mark.parametrize("k,eps", [(2, 1.0), (3, 0.5)])
def test_rank_4k_correction_reproduces_the_dense_mismatch(k, eps):
    t = _mismatch(k, eps)
    d = t.shape[0]
    assert np.allclose(t @ t.T, np.eye(d), atol=1e-12)              # still a rotation
    sigma = np.linalg.svd(t - np.eye(d), compute_uv=False)
    assert np.sum(sigma > 1e-9 * sigma[0]) <= 4 * k
    r = 4 * k
    u, _ = prep.principal_subspace(t, r)
    m = prep.subspace_transform(t, u)
    assert np.abs(prep.approx_operator(u, m) - t).max() < 1e-12
    h = np.random.default_rng(5).standard_normal((9, d))
    hc = online.reproject(h, online.transform(online.project(h, u), m), u)   # the oracle's steps, unrounded
    assert np.linalg.norm(hc - h @ t) <= 1e-12 * np.linalg.norm(h @ t)


def test_error_falls_with_rank_and_vanishes_at_4k():
    k, eps = 3, 1.0
    t = _mismatch(k, eps)
    d = t.shape[0]
    h = np.random.default_rng(6).standard_normal((16, d))
    ref = h @ t
    errs = []
    for r in (0, 2, 4, 8, 12):
        if r == 0:
            approx = h
        else:
            u, _ = prep.principal_subspace(t, r)
            approx = h @ prep.approx_operator(u, prep.subspace_transform(t, u))
        errs.append(np.linalg.norm(approx - ref) / np.linalg.norm(ref))
    assert all(b <= a + 1e-12 for a, b in zip(errs, errs[1:]))
    assert errs[0] > 1e-2 and errs[-1] < 1e-12
