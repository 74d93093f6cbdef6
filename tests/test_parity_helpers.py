"""The GPU parity helpers themselves (CPU only): the activation-code check must
accept differences only at rounding ties of the quantiser, and the bf16
regression bar must equal the rounding the oracle's own bf16 output carries."""
import numpy as np

from oracle import online
from oracle.numerics import round_to_bf16
from gpu_helpers import bf16_rounding_error, code_mismatch_ok


def _case(values, scale=1.0):
    a = np.asarray(values, np.float32)[None, :]
    s = np.asarray([scale], np.float32)
    ref = np.clip(np.rint(a / s[:, None]), -7, 7).astype(np.int64)
    return a, s, ref


def test_identical_codes_pass():
    a, s, ref = _case(np.linspace(-7, 7, 64))
    ok, nbad, dmax, nontie = code_mismatch_ok(ref.copy(), ref, a, s)
    assert ok and nbad == 0 and dmax == 0 and nontie == 0


def test_a_flip_at_an_exact_tie_passes():
    vals = np.zeros(20000, np.float32)
    vals[0] = 2.5                          # exactly half-way between codes 2 and 3
    a, s, ref = _case(vals)
    gpu = ref.copy()
    gpu[0, 0] = 3                          # rint(2.5) = 2 (ties to even); the other neighbour
    ok, nbad, dmax, nontie = code_mismatch_ok(gpu, ref, a, s)
    assert ok and nbad == 1 and nontie == 0


def test_a_flip_a_few_ulps_from_a_tie_passes_but_not_far_from_one():
    vals = np.zeros(20000, np.float32)
    vals[0] = np.nextafter(np.float32(2.5), np.float32(3), dtype=np.float32)   # one ulp above the tie
    vals[1] = np.float32(2.3)
    a, s, ref = _case(vals)
    gpu = ref.copy()
    gpu[0, 0] -= 1                        # 3 -> 2: a one-ulp flip of the statistics
    assert code_mismatch_ok(gpu, ref, a, s)[0]
    gpu[0, 1] += 1                        # 2 -> 3 at a / s = 2.3: a real error
    ok, _, _, nontie = code_mismatch_ok(gpu, ref, a, s)
    assert not ok and nontie == 1


def test_two_levels_or_too_many_ties_fail():
    vals = np.zeros(100, np.float32)
    vals[:3] = 0.5
    a, s, ref = _case(vals)
    gpu = ref.copy()
    gpu[0, 0] += 2
    assert not code_mismatch_ok(gpu, ref, a, s, max_frac=1.0)[0]
    gpu = ref.copy()
    gpu[0, :3] += 1                       # three tie flips in 100 codes: above 1e-4
    assert not code_mismatch_ok(gpu, ref, a, s)[0]
    assert code_mismatch_ok(gpu, ref, a, s, max_frac=0.05)[0]


def test_a_zero_row_admits_no_difference():
    a = np.zeros((1, 64), np.float32)
    s = np.zeros(1, np.float32)
    ref = np.zeros((1, 64), np.int64)
    gpu = ref.copy()
    gpu[0, 5] = 1
    assert not code_mismatch_ok(gpu, ref, a, s, max_frac=1.0)[0]


def test_bf16_rounding_error_is_the_rounding_of_the_exact_correction():
    rng = np.random.default_rng(3)
    d, r = 128, 4
    h = round_to_bf16(rng.standard_normal((6, d))).astype(np.float32)
    u = np.linalg.qr(rng.standard_normal((d, r)))[0].astype(np.float32)
    m = (0.3 * rng.standard_normal((r, r))).astype(np.float32)
    e = bf16_rounding_error(h, u, m)
    # bf16 keeps 8 significant bits: the relative rounding error lies below 2^-8
    assert 0 < e < 2.0 ** -8
    # with M = 0 the exact correction is h itself, already bf16: nothing to round
    assert bf16_rounding_error(h, u, np.zeros((r, r), np.float32)) == 0.0
    assert np.array_equal(online.correct(h, u, np.zeros((r, r), np.float32), "bf16"), h)
