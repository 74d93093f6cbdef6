"""Pins of the oracle's online steps (CPU only).

Correction: T = I identity, rank-D equals dense h T, error non-increasing in
r, T_hat orthogonal (norm preserved), linearity, worked 2-D and embedded-plane
cases. Norm: closed form of mean(a^2). Quantiser: brute force, symmetry,
scale invariance, worked examples. Packing: hand-worked bytes, round trips.
GEMM and dequantisation: brute force, closed forms and an error bound.
"""
import os

import numpy as np
import pytest

from oracle import online, packing, prep
from oracle.numerics import round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _skew(d, seed):
    g = np.random.default_rng(seed).standard_normal((d, d))
    u = np.triu(g, 1)
    return u - u.T


def _mismatch(d, seed, eps=0.05):
    return prep.basis_mismatch(prep.rotation(_skew(d, seed), eps), prep.rotation(_skew(d, seed + 1), eps))


def _bf16_exact(x):
    return round_to_bf16(x)


# ------------------------------------------------------------ correction
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_transform_is_bit_exact_identity(dtype):
    rng = np.random.default_rng(0)
    h = rng.standard_normal((9, 64)) * 30
    h = _bf16_exact(h) if dtype == "bf16" else h.astype(np.float32)
    u, _ = np.linalg.qr(rng.standard_normal((64, 8)))
    out = online.correct(h, u.astype(np.float32), np.zeros((8, 8), np.float32), dtype)
    assert np.array_equal(np.asarray(out, np.float64), np.asarray(h, np.float64))


def test_global_rotation_site_is_identity():
    # R_in = R_out: T = I, so the correction must hand back h unchanged (it §2B, nl §2B).
    d, r = 64, 8
    a = _skew(d, 1)
    t = prep.basis_mismatch(prep.rotation(a, 0.02), prep.rotation(a, 0.02))
    u, _ = prep.principal_subspace(t, r, check_gap=False)
    m = prep.subspace_transform(t, u)
    h = _bf16_exact(np.random.default_rng(1).standard_normal((5, d)))
    out = online.correct(h, u.astype(np.float32), m.astype(np.float32), "bf16")
    assert np.array_equal(out, h)


def test_rank_d_equals_dense_product():
    d = 64
    t = _mismatch(d, 2, 0.1)
    u, _ = prep.principal_subspace(t, d)
    m = prep.subspace_transform(t, u)
    h = np.random.default_rng(2).standard_normal((7, d))
    exact = online.reproject(h, online.transform(online.project(h, u), m), u)
    assert np.allclose(exact, h @ t, atol=1e-12)
    # with float32 inputs U_r, M the float32 output stays within 1e-5 relative L2
    out = online.correct(h, u.astype(np.float32), m.astype(np.float32), "f32").astype(np.float64)
    assert np.linalg.norm(out - h @ t) / np.linalg.norm(h @ t) < 1e-5


def test_error_non_increasing_in_rank():
    d = 128
    t = _mismatch(d, 3, 0.05)
    h = np.random.default_rng(3).standard_normal((16, d))
    u_all, _ = prep.principal_subspace(t, d)
    prev = None
    for r in (8, 16, 32, 64, d):
        u = u_all[:, :r]
        hp = online.reproject(h, online.transform(online.project(h, u), prep.subspace_transform(t, u)), u)
        err = np.linalg.norm(hp - h @ t, axis=1)
        if prev is not None:
            assert np.all(err <= prev * (1 + 1e-9) + 1e-12)
        prev = err
    assert np.max(prev) < 1e-10


def test_float32_operator_is_orthogonal_and_norm_preserving():
    d, r = 256, 32
    t = _mismatch(d, 4, 0.02)
    u, _ = prep.principal_subspace(t, r)
    m = prep.subspace_transform(t, u)
    u32, m32 = u.astype(np.float32).astype(np.float64), m.astype(np.float32).astype(np.float64)
    t_hat = prep.approx_operator(u32, m32)
    assert np.max(np.abs(t_hat.T @ t_hat - np.eye(d))) < 1e-5
    h = np.random.default_rng(4).standard_normal((32, d))
    hp = online.reproject(h, online.transform(online.project(h, u32), m32), u32)
    assert np.allclose(np.linalg.norm(hp, axis=1), np.linalg.norm(h, axis=1), rtol=1e-6)


def test_linearity():
    d, r = 64, 8
    t = _mismatch(d, 5)
    u, _ = prep.principal_subspace(t, r)
    m = prep.subspace_transform(t, u)
    rng = np.random.default_rng(5)
    h1, h2 = rng.standard_normal((3, d)), rng.standard_normal((3, d))
    f = lambda h: online.reproject(h, online.transform(online.project(h, u), m), u)  # noqa: E731
    assert np.allclose(f(2.5 * h1 - 0.75 * h2), 2.5 * f(h1) - 0.75 * f(h2), atol=1e-12)


def test_two_dimensional_rotation_worked_case():
    theta = 0.3
    c, s = np.cos(theta), np.sin(theta)
    t = np.array([[c, -s], [s, c]])
    u, sig = prep.principal_subspace(t, 2)
    assert np.allclose(sig, [2 * np.sin(theta / 2)] * 2, atol=1e-14)
    m = prep.subspace_transform(t, u)
    h = np.array([[1.0, 2.0]])
    out = online.reproject(h, online.transform(online.project(h, u), m), u)
    assert np.allclose(out, [[1.0 * c + 2.0 * s, -1.0 * s + 2.0 * c]], atol=1e-14)


def test_single_embedded_plane_is_captured_exactly_at_rank_two():
    theta = 0.7
    c, s = np.cos(theta), np.sin(theta)
    t = np.eye(4)
    t[1:3, 1:3] = [[c, -s], [s, c]]
    u, sig = prep.principal_subspace(t, 2)
    assert np.allclose(sig[2:], 0, atol=1e-14)
    assert np.allclose(prep.approx_operator(u, prep.subspace_transform(t, u)), t, atol=1e-14)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_mean_square_closed_form():
    rng = np.random.default_rng(6)
    x = _bf16_exact(rng.standard_normal((10, 256)) * 3)
    eps = 1e-5
    a = online.rmsnorm(x, eps).astype(np.float64)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(a * a, axis=1), ms / (ms + eps), rtol=1e-6)


def test_rmsnorm_scale_invariance_without_eps():
    x = np.random.default_rng(7).standard_normal((4, 128)).astype(np.float32)
    assert np.array_equal(online.rmsnorm(x, 0.0), online.rmsnorm(x * np.float32(8.0), 0.0))


def test_rmsnorm_weight_multiplies_after_normalisation():
    x = np.random.default_rng(8).standard_normal((3, 64)).astype(np.float32)
    w = np.random.default_rng(9).standard_normal(64).astype(np.float32)
    assert np.array_equal(online.rmsnorm(x, 1e-5, w), online.rmsnorm(x, 1e-5) * w)


# -------------------------------------------------------------- quantiser
def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c.strip() for c in line.split("|")])
    return rows


def test_quantiser_worked_examples():
    for bits, a, s, q in _read_table("quant_worked.txt"):
        a = np.array([float(v) for v in a.split(",")], np.float32)
        codes, scale = online.quantize(a, int(bits))
        assert np.float32(s) == scale[0]
        assert codes[0].tolist() == [int(v) for v in q.split(",")]


def _brute_force_codes(a, s, qm):
    # the nearest level q*s over all q in [-qmax, qmax]; equidistant: the even q
    cand = np.arange(-qm, qm + 1)
    out = []
    for v in a:
        dist = np.abs(np.float32(v) / np.float32(s) - cand.astype(np.float64))
        best = np.flatnonzero(dist == dist.min())
        out.append(int(cand[best[0]]) if len(best) == 1 else int(cand[best][cand[best] % 2 == 0][0]))
    return out


@pytest.mark.parametrize("bits", [3, 4])
def test_quantiser_matches_brute_force(bits):
    rng = np.random.default_rng(10 + bits)
    qm = packing.qmax(bits)
    for trial in range(200):
        n = rng.integers(1, 9)
        a = (rng.standard_normal(n) * 10 ** rng.uniform(-3, 3)).astype(np.float32)
        if trial % 5 == 0:  # plant exact half-level ties
            s0 = np.float32(0.25)
            a = (rng.integers(-2 * qm, 2 * qm + 1, n) * s0 / 2).astype(np.float32)
            a[0] = qm * s0
        codes, s = online.quantize(a, bits)
        assert codes[0].tolist() == _brute_force_codes(a, s[0], qm)
        assert np.max(np.abs(codes)) == (qm if np.any(a != 0) else 0)


@pytest.mark.parametrize("bits", [3, 4])
def test_quantiser_symmetry_and_power_of_two_invariance(bits):
    a = np.random.default_rng(20).standard_normal((6, 96)).astype(np.float32)
    q, s = online.quantize(a, bits)
    qn, sn = online.quantize(-a, bits)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    q2, s2 = online.quantize(a * np.float32(2.0 ** -5), bits)
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** -5))


def test_quantiser_zero_row():
    q, s = online.quantize(np.zeros((2, 64), np.float32), 4)
    assert not q.any() and not s.any()


# ---------------------------------------------------------------- packing
def test_packing_hand_worked_bytes():
    for bits, codes, expect in _read_table("packing_bytes.txt"):
        codes = np.array([[int(v) for v in codes.split(",")]])
        got = packing.pack(codes, int(bits))[0]
        assert got.tolist() == [int(b, 16) for b in expect.split()], (bits, codes)
        assert np.array_equal(packing.unpack(got[None, :], codes.shape[1], int(bits)), codes)


@pytest.mark.parametrize("bits", [3, 4])
def test_packing_round_trip_all_values(bits):
    rng = np.random.default_rng(30 + bits)
    qm = packing.qmax(bits)
    codes = rng.integers(-qm - 1, qm + 1, size=(17, 256))
    p = packing.pack(codes, bits)
    assert p.shape == (17, packing.packed_row_bytes(256, bits))
    assert np.array_equal(packing.unpack(p, 256, bits), codes)


def test_int3_packing_single_code_positions():
    # a single nonzero code lands in the bits its slot and lane name, nowhere else
    for i in range(32):
        codes = np.zeros((1, 32), np.int64)
        codes[0, i] = -1                                    # pattern 111
        p = packing.pack(codes, 3)[0].astype(np.int64)
        j, b = divmod(i, 4)
        assert bin(int(sum(int(x) << (8 * k) for k, x in enumerate(p)))).count("1") == 3
        if j < 6:
            assert p[4 * (j // 2) + b] == (0xE0 if j % 2 == 0 else 0x1C)
        else:
            assert p[4 * (j - 6) + b] == 0x03
            assert p[8 + b] == (0x02 if j == 6 else 0x01)


def test_packing_rejects_bad_width():
    with pytest.raises(ValueError):
        packing.pack(np.zeros((1, 33), np.int64), 3)
    with pytest.raises(ValueError):
        packing.pack(np.zeros((1, 3), np.int64), 4)


# ------------------------------------------------------------- GEMM, dequant
def test_gemm_matches_triple_loop():
    rng = np.random.default_rng(40)
    qa, qw = rng.integers(-7, 8, (5, 64)), rng.integers(-7, 8, (6, 64))
    acc = online.gemm(qa, qw)
    for t in range(5):
        for j in range(6):
            assert acc[t, j] == sum(int(qa[t, k]) * int(qw[j, k]) for k in range(64))


def test_gemm_all_ones_weight_gives_row_sums():
    qa = np.random.default_rng(41).integers(-7, 8, (4, 128))
    acc = online.gemm(qa, np.ones((3, 128), np.int64))
    assert np.array_equal(acc, np.repeat(qa.sum(axis=1)[:, None], 3, axis=1))


def test_gemm_extreme_codes_fit_int32():
    k = 28672
    acc = online.gemm(np.full((1, k), -7), np.full((1, k), -7))
    assert acc[0, 0] == 49 * k < 2 ** 31


def test_dequant_equals_scaled_float64_sum():
    rng = np.random.default_rng(42)
    qa, qw = rng.integers(-7, 8, (6, 256)), rng.integers(-7, 8, (5, 256))
    sa = rng.uniform(0.01, 1, 6).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, 5).astype(np.float32)
    y = online.dequant(online.gemm(qa, qw), sa, sw, "f32").astype(np.float64)
    ref = (qa * sa[:, None].astype(np.float64)) @ (qw * sw[:, None].astype(np.float64)).T
    assert np.all(np.abs(y - ref) <= 4 * np.spacing(np.abs(y).astype(np.float32)).astype(np.float64) + 1e-30)


def test_quantised_linear_error_bound():
    rng = np.random.default_rng(43)
    k = 256
    a = rng.standard_normal((8, k)).astype(np.float32)
    w = (rng.standard_normal((16, k)) * 0.02).astype(np.float32)
    qa, sa = online.quantize(a, 4)
    qw, sw = prep.quantize_weight(w, 4)
    y = online.dequant(online.gemm(qa, qw), sa, sw, "f32").astype(np.float64)
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    bound = (np.abs(a) @ (sw[:, None] / 2 * np.ones((1, k))).T
             + (sa[:, None] / 2) * np.abs(w).sum(axis=1)[None, :]
             + k * sa[:, None] * sw[None, :] / 4)
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-6) + 1e-6 * np.abs(exact))


def test_packed_linear_matches_unpacked():
    rng = np.random.default_rng(44)
    for bits in (3, 4):
        qm = packing.qmax(bits)
        qa, qw = rng.integers(-qm, qm + 1, (4, 64)), rng.integers(-qm, qm + 1, (8, 64))
        sa, sw = rng.uniform(0.1, 1, 4).astype(np.float32), rng.uniform(0.1, 1, 8).astype(np.float32)
        y, acc = online.qgemm_packed(packing.pack(qa, bits), sa, packing.pack(qw, bits), sw, 64, bits, "f32")
        assert np.array_equal(acc, online.gemm(qa, qw))
        assert np.array_equal(y, online.dequant(acc, sa, sw, "f32"))


# --------------------------------------------------------------- rounding
def test_bf16_rounding_worked_values():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    assert round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert round_to_bf16(np.array([1 + 2 ** -8 + 2 ** -30]))[0] == 1 + 2 ** -7
    assert round_to_bf16(np.array([-3.0]))[0] == -3.0
    x = np.random.default_rng(45).standard_normal(1000)
    r = round_to_bf16(x)
    # every result has at most 8 significant bits and lies within half a bf16 ulp
    m, e = np.frexp(r)
    assert np.array_equal(np.ldexp(m, 8), np.rint(np.ldexp(m, 8)))
    assert np.all(np.abs(r - x) <= np.ldexp(1.0, np.frexp(x)[1] - 9) * (1 + 1e-12))


# ------------------------------------------------------------ residual add
def test_dequant_add_with_zero_residual_is_dequant():
    rng = np.random.default_rng(44)
    acc = online.gemm(rng.integers(-7, 8, (5, 96)), rng.integers(-7, 8, (7, 96)))
    sa = rng.uniform(0.01, 1, 5).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, 7).astype(np.float32)
    for dt in ("f32", "bf16"):
        assert np.array_equal(online.dequant_add(acc, sa, sw, np.zeros((5, 7), np.float32), dt),
                              online.dequant(acc, sa, sw, dt))


def test_dequant_add_with_zero_codes_returns_the_residual():
    rng = np.random.default_rng(45)
    r = round_to_bf16(rng.standard_normal((4, 32)) * 10)
    y = online.dequant_add(np.zeros((4, 32), np.int64), np.ones(4, np.float32), np.ones(32, np.float32), r, "bf16")
    assert np.array_equal(y, r)


def test_dequant_add_within_three_roundings_of_the_exact_sum():
    rng = np.random.default_rng(46)
    acc = online.gemm(rng.integers(-7, 8, (6, 128)), rng.integers(-7, 8, (9, 128)))
    sa = rng.uniform(0.01, 1, 6).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, 9).astype(np.float32)
    r = rng.standard_normal((6, 9)).astype(np.float32)
    y = online.dequant_add(acc, sa, sw, r, "f32").astype(np.float64)
    v = acc * sa[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    exact = v + r
    # two roundings inside v (relative to |v|), one of the sum (relative to |y|)
    ulp = lambda x: np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)  # noqa: E731
    assert np.all(np.abs(y - exact) <= 2 * ulp(v) + ulp(y))


def _chain_inputs(d=64, f=96, n=6, seed=47):
    rng = np.random.default_rng(seed)
    h = round_to_bf16(rng.standard_normal((n, d)))
    o_in = round_to_bf16(rng.standard_normal((n, d)))
    down_in = round_to_bf16(rng.standard_normal((n, f)))

    def lin(nout, k, zero=False):
        w = np.zeros((nout, k), np.float32) if zero else (rng.standard_normal((nout, k)) * 0.05).astype(np.float32)
        q, s = prep.quantize_weight(w, 4)
        return packing.pack(q, 4), s
    return h, o_in, down_in, lin


def test_layer_chain_with_identity_sites_and_zero_outputs_keeps_the_residual():
    d, f = 64, 96
    h, o_in, down_in, lin = _chain_inputs(d, f)
    u = np.linalg.qr(np.random.default_rng(48).standard_normal((d, 2)))[0].astype(np.float32)
    site = (u, np.zeros((2, 2), np.float32))
    weights = {"qkv": lin(3 * d, d), "o": lin(d, d, zero=True), "gate_up": lin(2 * f, d), "down": lin(d, f, zero=True)}
    out = online.layer_chained(h, site, site, weights, o_in, down_in, "bf16", 4, 1e-5, "bf16")
    assert np.array_equal(out["h2"], h) and np.array_equal(out["h3"], h)


def test_layer_chain_carries_each_residual_add_into_the_next_site():
    d, f = 64, 96
    h, o_in, down_in, lin = _chain_inputs(d, f, seed=49)
    u = np.linalg.qr(np.random.default_rng(50).standard_normal((d, 2)))[0].astype(np.float32)
    site = (u, np.zeros((2, 2), np.float32))
    weights = {"qkv": lin(3 * d, d), "o": lin(d, d), "gate_up": lin(2 * f, d), "down": lin(d, f)}
    out = online.layer_chained(h, site, site, weights, o_in, down_in, "bf16", 4, 1e-5, "bf16")
    # identity sites: h2 = bf16(h + o(o_in)), site B sees h2, h3 = bf16(h2 + down(down_in))
    o_y = online.qgemm_packed(*online.quant_act_packed(o_in, 4, False)[:2], *weights["o"], d, 4, "f32")[0]
    d_y = online.qgemm_packed(*online.quant_act_packed(down_in, 4, False)[:2], *weights["down"], f, 4, "f32")[0]
    h2 = round_to_bf16(o_y.astype(np.float32) + h.astype(np.float32))
    assert np.array_equal(out["h2"], h2)
    assert np.array_equal(out["siteB"]["h_out"], h2)
    assert np.array_equal(out["h3"], round_to_bf16(d_y.astype(np.float32) + h2.astype(np.float32)))


# ------------------------------------------------------------ fp4 codes
def _fp4_fixture():
    values, rows = {}, []
    with open(os.path.join(GOLDEN, "fp4_bytes.txt")) as fh:
        text = fh.read()
    for line in text.splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        left, right = (x.strip() for x in line.split("|"))
        if "=" not in left:
            values[int(left, 16)] = float(right)
            continue
        codes = np.zeros((1, 32), np.int64)
        for item in left.split(","):
            idx, val = item.split("=")
            if idx == "all":
                codes[:] = int(val)
            else:
                codes[0, int(idx)] = int(val)
        rows.append((codes, [int(b, 16) for b in right.split()]))
    return values, rows


def test_e2m1_values_match_the_mx_table():
    values, _ = _fp4_fixture()
    assert sorted(values) == list(range(8))
    for pat, v in values.items():
        assert packing.e2m1_value(pat) == v
        assert packing.e2m1_value(pat | 8) == -v


def test_fp4_packing_hand_worked_bytes():
    _, rows = _fp4_fixture()
    assert len(rows) >= 5
    for codes, expect in rows:
        got = packing.pack_fp4(codes)[0]
        assert got.tolist() == expect, codes
        assert np.array_equal(packing.unpack_fp4(got[None, :], 32), codes)


def test_fp4_round_trip_and_same_codes_as_int3():
    rng = np.random.default_rng(44)
    codes = rng.integers(-3, 4, size=(9, 160))
    p = packing.pack_fp4(codes)
    assert p.shape == (9, 80)
    assert np.array_equal(packing.unpack_fp4(p, 160), codes)
    assert np.array_equal(packing.unpack(packing.pack(codes, 3), 160, 3), packing.unpack_fp4(p, 160))
    # every code is exact: twice the element value is the code
    assert all(2 * packing.e2m1_value(packing.pack_fp4(np.full((1, 32), c))[0, 0] >> 4) == c for c in range(-3, 4))


def test_fp4_rejects_codes_outside_the_3bit_range():
    with pytest.raises(ValueError):
        packing.pack_fp4(np.full((1, 32), -4))
    with pytest.raises(ValueError):
        packing.unpack_fp4(np.full((1, 16), 0x44, np.uint8), 32)   # 2.0 -> code 4


# ------------------------------------------------ one site and its linear, M != 0
def _quarter_turn_site(d, i=0, j=1):
    """The site of a quarter turn in the plane of coordinates i and j: U = [e_i e_j],
    M = R - I_2 with R the 90-degree rotation. For a row h its exact correction is
    h with (h_i, h_j) replaced by (h_j, -h_i); every float64 step is exact."""
    u = np.zeros((d, 2), np.float32)
    u[i, 0] = u[j, 1] = 1.0
    rot = np.array([[0.0, -1.0], [1.0, 0.0]])
    return u, (rot - np.eye(2)).astype(np.float32)


def _turned(x, i=0, j=1):
    y = np.array(x, copy=True)
    y[:, i], y[:, j] = x[:, j], -x[:, i]
    return y


def test_layer_fused_with_a_quarter_turn_site():
    # zh 2.2 steps 1-3 with a non-identity M whose result is known exactly; the
    # norm and the quantiser are invariant under the turn (same multiset of
    # magnitudes), so the codes are the turned codes of h, and the linear
    # equals the plain linear with the weight's columns 0 and 1 turned back.
    rng = np.random.default_rng(60)
    d, n, nout, bits = 64, 7, 32, 4
    h = rng.standard_normal((n, d)) * 3
    h[:, 5] *= 40                                              # an outlier channel
    h = _bf16_exact(h)
    u, m = _quarter_turn_site(d)
    w = (rng.standard_normal((nout, d)) * 0.02).astype(np.float32)
    qw, sw = prep.quantize_weight(w, bits)
    out = online.layer_fused(h, u, m, "bf16", bits, 1e-5, packing.pack(qw, bits), sw, "bf16")
    assert np.array_equal(out["h_out"], _turned(h))
    assert not np.array_equal(out["h_out"], h)
    q_plain, s_plain = online.quant_act(h, bits, True, 1e-5)
    assert np.array_equal(out["q"], _turned(q_plain))
    assert np.array_equal(out["scales"], s_plain)
    # sum_k q'_k w_k = q1 w0 - q0 w1 + ... = sum_k q_k w''_k with w''_0 = -w_1, w''_1 = w_0
    qw_back = np.array(qw, copy=True)
    qw_back[:, 0], qw_back[:, 1] = -qw[:, 1], qw[:, 0]
    y_plain, acc_plain = online.qgemm_packed(packing.pack(q_plain, bits), s_plain, packing.pack(qw_back, bits), sw,
                                             d, bits, "bf16")
    assert np.array_equal(out["acc"], acc_plain)
    assert np.array_equal(out["y"], y_plain)


def _constant_linear(nout, k, code, bits):
    """Packed weight codes all equal to `code`, unit channel scales."""
    return packing.pack(np.full((nout, k), code, np.int64), bits), np.ones(nout, np.float32)


def test_layer_linear_path_wires_each_linear_to_its_input():
    # The path of one layer: site A corrects h and feeds q|k|v, site B corrects
    # site A's h' and feeds gate|up, o reads the o_proj input and down the
    # down_proj input. Both sites are quarter turns (in different planes), so
    # each corrected residual and its codes are known exactly; constant weights
    # turn each output into a closed form of its input's codes (a row sum),
    # different for every linear, so any miswiring shows.
    rng = np.random.default_rng(61)
    d, f, n, bits = 64, 96, 5, 4
    h = _bf16_exact(rng.standard_normal((n, d)) * 2)
    o_in = _bf16_exact(rng.standard_normal((n, d)))
    down_in = _bf16_exact(rng.standard_normal((n, f)))
    site_a, site_b = _quarter_turn_site(d, 0, 1), _quarter_turn_site(d, 2, 3)
    weights = {"qkv": _constant_linear(3 * d, d, 1, bits), "o": _constant_linear(d, d, 2, bits),
               "gate_up": _constant_linear(2 * f, d, -1, bits), "down": _constant_linear(d, f, 3, bits)}
    out = online.layer_linear_path(h, site_a, site_b, weights, o_in, down_in, "bf16", bits, 1e-5, "f32")
    h_a, h_b = _turned(h, 0, 1), _turned(_turned(h, 0, 1), 2, 3)
    assert np.array_equal(out["siteA"]["h_out"], h_a)
    assert np.array_equal(out["siteB"]["h_out"], h_b)            # site B's input is site A's h'
    q_plain, s_plain = online.quant_act(h, bits, True, 1e-5)      # the turns keep the norm and the scale
    qa, sa = out["siteA"]["q"], out["siteA"]["scales"]
    qb, sb = out["siteB"]["q"], out["siteB"]["scales"]
    assert np.array_equal(qa, _turned(q_plain, 0, 1)) and np.array_equal(sa, s_plain)
    assert np.array_equal(qb, _turned(_turned(q_plain, 0, 1), 2, 3)) and np.array_equal(sb, s_plain)

    def row_sum_output(q, s, code, nout):
        v = (q.sum(axis=1).astype(np.float32) * code) * s       # (float32(acc) * s_a) * s_w with s_w = 1
        return np.repeat(v[:, None].astype(np.float32), nout, axis=1)
    qo, so = online.quant_act(o_in, bits, False)
    qd, sd = online.quant_act(down_in, bits, False)
    assert np.array_equal(out["qkv"], row_sum_output(qa, sa, 1, 3 * d))
    assert np.array_equal(out["gate_up"], row_sum_output(qb, sb, -1, 2 * f))
    assert np.array_equal(out["o"], row_sum_output(qo, so, 2, d))
    assert np.array_equal(out["down"], row_sum_output(qd, sd, 3, d))
    # the row sums of the two sites' codes differ, so swapping their linears would show
    assert not np.array_equal(qa.sum(axis=1), qb.sum(axis=1))
