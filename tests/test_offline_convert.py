"""The library's offline site conversion against the oracle's prep (CPU only).

The two are written independently (the library takes the top eigenspace of
2I - T - T^T with a partial symmetric eigensolver and builds Hadamard from
bit parities; the oracle uses a full SVD of T - I and the Sylvester
recursion), so agreement of the applied operator I + U M U^T pins both.
"""
import numpy as np
import pytest

import synth
from oracle import prep
from rotation_bit_post_amd import offline


@pytest.mark.parametrize("d", [2, 8, 64, 256])
def test_hadamard_constructions_agree(d):
    assert np.allclose(offline.sylvester_hadamard(d), prep.hadamard(d), atol=1e-15)


@pytest.mark.parametrize("d,r,eps", [(64, 8, 0.05), (256, 32, 0.02), (256, 8, 0.02), (128, 64, 0.1)])
def test_site_operator_matches_oracle(d, r, eps):
    rng = np.random.default_rng(d + r)
    g1, g2 = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    a_in, a_out = np.triu(g1, 1) - np.triu(g1, 1).T, np.triu(g2, 1) - np.triu(g2, 1).T
    U, M = offline.convert_site(offline.synthetic_rotation(a_in, eps), offline.synthetic_rotation(a_out, eps), r)
    ref = prep.site(a_in, a_out, eps, r)
    op = prep.approx_operator(U.astype(np.float64), M.astype(np.float64))
    op_ref = prep.approx_operator(ref["U"], ref["M"])
    assert np.max(np.abs(op - op_ref)) < 1e-6          # float32 rounding of U and M
    assert np.allclose(U.T.astype(np.float64) @ U, np.eye(r), atol=1e-6)


def test_tiny_site_matches_oracle():
    cfg = synth.WORKLOADS[synth.TINY]
    a_in, a_out = synth.skew_generator(cfg, "A", "in"), synth.skew_generator(cfg, "A", "out")
    U, M = offline.convert_site(offline.synthetic_rotation(a_in, cfg.eps_rot),
                                offline.synthetic_rotation(a_out, cfg.eps_rot), cfg.r)
    ref = prep.site(a_in, a_out, cfg.eps_rot, cfg.r)
    assert np.max(np.abs(prep.approx_operator(U.astype(np.float64), M.astype(np.float64))
                         - prep.approx_operator(ref["U"], ref["M"]))) < 1e-6


def test_convert_rejects_a_rank_inside_a_pair():
    rng = np.random.default_rng(1)
    g = rng.standard_normal((32, 32))
    a = np.triu(g, 1) - np.triu(g, 1).T
    g2 = rng.standard_normal((32, 32))
    b = np.triu(g2, 1) - np.triu(g2, 1).T
    with pytest.raises(ValueError):
        offline.convert_site(offline.cayley_rotation(a, 0.1), offline.cayley_rotation(b, 0.1), 5)
