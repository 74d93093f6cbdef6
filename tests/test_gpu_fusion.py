"""GPU parity of the offline weight fusion (rsq_rotate_weight) against the
oracle's float64 fusion. Both sides form the same exact float64 products and
sum them in float64 in different orders, so the two sums differ by at most
2 (K - 1) 2^-53 sum|w_i r_i|, and their float32 roundings by that plus one
float32 ulp. The per-channel weight codes of the fused weight equal the
oracle's except at rounding ties."""
import numpy as np
import pytest

import synth
from oracle import packing, prep
from gpu_helpers import code_mismatch_ok, empty_f32, empty_u8, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _orth(d, seed, eps=0.05):
    g = np.random.default_rng(seed).standard_normal((d, d))
    a = np.triu(g, 1)
    return prep.cayley(eps * (a - a.T)).astype(np.float32)


def _beyond_sum_order_bound(got, ref, abs_sum, k):
    """Outputs farther apart than one float32 ulp plus the float64 summation-order bound."""
    got, ref = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    ulp = np.spacing(np.maximum(np.abs(got), np.abs(ref))).astype(np.float64)
    bound = ulp + 2.0 * (k - 1) * 2.0 ** -53 * abs_sum
    bad = np.abs(got.astype(np.float64) - ref.astype(np.float64)) > bound
    return int(np.sum(bad)), int(np.sum(got != ref))


@pytest.mark.parametrize("n,k", [(64, 96), (96, 64), (32, 2048), (160, 224)])
def test_rotate_weight_matches_oracle(n, k):
    import torch
    rsq = lib()
    from rotation_bit_post_amd.offline_device import fuse_weight_device
    print(f"case rotate n={n} k={k}", flush=True)
    w = (np.random.default_rng(n + k).standard_normal((n, k)) * 0.02).astype(np.float32)
    r_in, r_out = _orth(k, 1), _orth(n, 2)
    got_r = fuse_weight_device(to_dev(w, "f32"), right=to_dev(r_in, "f32"))
    got_l = fuse_weight_device(to_dev(w, "f32"), left=to_dev(r_out, "f32"))
    got_2 = fuse_weight_device(to_dev(w, "f32"), right=to_dev(r_in, "f32"), left=to_dev(r_out, "f32"))
    torch.cuda.synchronize()
    a64 = lambda x: np.abs(np.asarray(x, np.float64))  # noqa: E731
    # both sides: the left stage checked on the device's own right-fused weight (identical inputs)
    mid = got_r.cpu().numpy()
    cases = ((got_r, prep.fuse_weight(w, right=r_in), a64(w) @ a64(r_in), k),
             (got_l, prep.fuse_weight(w, left=r_out), a64(r_out).T @ a64(w), n),
             (got_2, prep.fuse_weight(mid, left=r_out), a64(r_out).T @ a64(mid), n))
    for got, ref, abs_sum, inner in cases:
        beyond, differ = _beyond_sum_order_bound(got.cpu().numpy(), ref, abs_sum, inner)
        print(f"  differing outputs {differ}, beyond one ulp {beyond}", flush=True)
        assert beyond == 0
    # the identity leaves the weight unchanged, bit for bit
    same = fuse_weight_device(to_dev(w, "f32"), right=to_dev(np.eye(k, dtype=np.float32), "f32"))
    torch.cuda.synchronize()
    assert np.array_equal(same.cpu().numpy(), w)
    assert rsq.RSQ_ROTATE_LEFT == 1


def test_q_projection_fused_with_the_workload_rotation_and_quantised():
    """The LLaMA-2-7B-shaped q projection (4096 x 4096) fused with site A's input
    rotation H C(eps A) on the device, then quantised per channel on the device."""
    import torch
    rsq = lib()
    from rotation_bit_post_amd.offline_device import fuse_weight_device
    cfg = synth.WORKLOADS[synth.LLAMA2_7B_PREFILL]
    print("case fused q projection 4096 x 4096", flush=True)
    w = synth.weight(cfg, "q", cfg.D, cfg.D)
    r = prep.rotation(synth.skew_generator(cfg, "A", "in"), cfg.eps_rot).astype(np.float32)
    got = fuse_weight_device(to_dev(w, "f32"), right=to_dev(r, "f32"))
    codes, scales = empty_u8(cfg.D, cfg.D // 2), empty_f32(cfg.D)
    rsq.rsq_quant_act(got, codes, scales, cfg.bits)
    torch.cuda.synchronize()
    ref = prep.fuse_weight(w, right=r)
    g = got.cpu().numpy()
    abs_sum = np.abs(w.astype(np.float64)) @ np.abs(r.astype(np.float64))
    beyond, differ = _beyond_sum_order_bound(g, ref, abs_sum, cfg.D)
    print(f"  differing outputs {differ} of {g.size}, beyond one ulp {beyond}", flush=True)
    assert beyond == 0
    q_ref, s_ref = prep.quantize_weight(ref, cfg.bits)
    q_gpu = packing.unpack(codes.cpu().numpy(), cfg.D, cfg.bits)
    s_gpu = scales.cpu().numpy()
    # the device codes against the oracle quantiser on the device's own fused weight: ties only
    q_own, s_own = prep.quantize_weight(g, cfg.bits)
    ok, nbad, _, nontie = code_mismatch_ok(q_gpu, q_own, g, s_gpu)
    assert ok, (nbad, nontie)
    assert np.all(np.abs(s_gpu - s_own) <= 1e-6 * s_own)
    # and against the oracle's fused weight: the scales within an ulp's effect
    assert np.all(np.abs(s_gpu - s_ref) <= 4e-7 * s_ref + 1e-30)
