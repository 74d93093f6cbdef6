"""Device offline conversion (torch float64; run here on the CPU back end)
against the oracle's SVD-based prep: same subspace, same operator."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import prep
from rotation_bit_post_amd.offline_device import convert_site_device, synthetic_rotation_device


def _operator(u, m):
    u = np.asarray(u, np.float64)
    return np.eye(u.shape[0]) + u @ np.asarray(m, np.float64) @ u.T


@pytest.mark.parametrize("r", [8, 16])
def test_device_conversion_matches_oracle_subspace_and_operator(r):
    cfg = synth.WORKLOADS[synth.TINY]
    a_in, a_out = synth.skew_generator(cfg, "A", "in"), synth.skew_generator(cfg, "A", "out")
    s = prep.site(a_in, a_out, cfg.eps_rot, r)
    r_in = synthetic_rotation_device(a_in, cfg.eps_rot, device="cpu")
    r_out = synthetic_rotation_device(a_out, cfg.eps_rot, device="cpu")
    u, m, iters, res = convert_site_device(r_in, r_out, r)
    assert res < 1e-9, (iters, res)
    # the same subspace: projectors agree
    pu = u.astype(np.float64) @ u.T.astype(np.float64)
    po = s["U"] @ s["U"].T
    assert np.max(np.abs(pu - po)) < 1e-5
    # the same approximate operator (float32 rounding of both)
    assert np.max(np.abs(_operator(u, m) - prep.approx_operator(s["U"], s["M"]))) < 1e-5


def test_device_rotation_equals_host_rotation():
    cfg = synth.WORKLOADS[synth.TINY]
    a = synth.skew_generator(cfg, "B", "in")
    r_dev = synthetic_rotation_device(a, cfg.eps_rot, device="cpu").numpy()
    assert np.max(np.abs(r_dev - prep.rotation(a, cfg.eps_rot))) < 1e-12


def test_device_conversion_refuses_a_rank_inside_a_pair():
    cfg = synth.WORKLOADS[synth.TINY]
    a_in, a_out = synth.skew_generator(cfg, "A", "in"), synth.skew_generator(cfg, "A", "out")
    r_in = synthetic_rotation_device(a_in, cfg.eps_rot, device="cpu")
    r_out = synthetic_rotation_device(a_out, cfg.eps_rot, device="cpu")
    with pytest.raises(ValueError):
        convert_site_device(r_in, r_out, 7)


def test_device_conversion_refuses_an_unconverged_subspace():
    cfg = synth.WORKLOADS[synth.TINY]
    a_in, a_out = synth.skew_generator(cfg, "A", "in"), synth.skew_generator(cfg, "A", "out")
    r_in = synthetic_rotation_device(a_in, cfg.eps_rot, device="cpu")
    r_out = synthetic_rotation_device(a_out, cfg.eps_rot, device="cpu")
    with pytest.raises(ValueError, match="did not converge"):
        convert_site_device(r_in, r_out, 8, max_iters=3)
