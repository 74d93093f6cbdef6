"""GPU parity of each C-ABI entry point against the oracle (small and ragged shapes).

Bars (taken in full from the method's stated tolerances): correction
outputs within relative L2 1e-3 (float32 residual) or 2e-2 (bfloat16
residual) of the float64 oracle; activation codes equal except at rounding
ties (at most one level, on at most 1e-4 of the elements); integer
accumulators bit-exact; dequantised outputs bit-exact when codes and scales
are identical (both sides then do the same float32 operations).
"""
import numpy as np
import pytest

from oracle import online, packing, prep
from oracle.numerics import round_to_bf16
from gpu_helpers import (bf16_rounding_error, code_mismatch_ok, empty_f32, empty_u8, lib, quant_input, rel_l2,
                         require_gpu, subspace_site, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _skew(d, seed):
    g = np.random.default_rng(seed).standard_normal((d, d))
    u = np.triu(g, 1)
    return u - u.T


def random_site(d, r, seed, eps=0.05):
    """(U32, M32) of a random mismatch T = C_out^T C_in (no Hadamard needed for any d)."""
    t = prep.cayley(eps * _skew(d, seed + 1)).T @ prep.cayley(eps * _skew(d, seed))
    u, _ = prep.principal_subspace(t, r)
    return u.astype(np.float32), prep.subspace_transform(t, u).astype(np.float32)


def residual(n, d, dtype, seed, outliers=3, scale=40.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, d)).astype(np.float32)
    h[:, rng.choice(d, min(outliers, d), replace=False)] *= scale
    return round_to_bf16(h).astype(np.float32) if dtype == "bf16" else h


def gpu_site(U, M):
    rsq = lib()
    import torch
    d, r = U.shape
    buf = torch.empty(rsq.rsq_site_bytes(d, r), dtype=torch.uint8, device="cuda")
    rsq.rsq_site_prepare(to_dev(U, "f32"), to_dev(M, "f32"), buf)
    return buf


CORRECT_CASES = [  # dtype, d, r, n
    ("f32", 256, 8, 16), ("f32", 256, 8, 3), ("bf16", 256, 8, 17), ("bf16", 96, 8, 7),
    ("bf16", 1024, 32, 33), ("bf16", 512, 64, 40), ("f32", 128, 16, 5), ("bf16", 2048, 2, 1),
    ("f32", 1024, 40, 19),
    ("f32", 4096, 32, 20),   # the widest float32 residual
    ("bf16", 8192, 64, 9),   # the widest residual at the largest rank (column-split form)
]


@pytest.mark.parametrize("dtype,d,r,n", CORRECT_CASES)
def test_subspace_correct_matches_oracle(dtype, d, r, n):
    rsq = lib()
    import torch
    print(f"case correct dtype={dtype} d={d} r={r} n={n}", flush=True)
    U, M = random_site(d, r, seed=d + r) if d <= 2048 else subspace_site(d, r, seed=d + r)
    h = residual(n, d, dtype, seed=n)
    site = gpu_site(U, M)
    hd = to_dev(h, dtype)
    out = torch.empty_like(hd)
    rsq.rsq_subspace_correct(hd, out, site, r)
    torch.cuda.synchronize()
    got = to_host(out).astype(np.float64)
    ref = np.asarray(online.correct(h, U, M, dtype), np.float64)
    err = rel_l2(got, ref)
    own = bf16_rounding_error(h, U, M) if dtype == "bf16" else 0.0
    print(f"  rel_l2={err:.3e} (oracle's own bf16 rounding {own:.3e})")
    assert err <= (1e-3 if dtype == "f32" else 2e-2)
    if dtype == "f32":
        assert err <= 1e-5
    else:   # regression bar: the bf16 operands cost no more than the rounding of h' itself
        assert err <= 2 * own
    # the float32 operator is orthogonal: row norms are preserved
    nr = np.linalg.norm(got, axis=1) / np.linalg.norm(h.astype(np.float64), axis=1)
    assert np.max(np.abs(nr - 1)) <= (1e-5 if dtype == "f32" else 4e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_transform_is_identity_and_in_place_works(dtype):
    rsq = lib()
    import torch
    d, r, n = 512, 32, 21
    U, _ = random_site(d, r, seed=3)
    h = residual(n, d, dtype, seed=4)
    site = gpu_site(U, np.zeros((r, r), np.float32))
    hd = to_dev(h, dtype)
    out = torch.empty_like(hd)
    rsq.rsq_subspace_correct(hd, out, site, r)
    torch.cuda.synchronize()
    assert torch.equal(out, hd)
    # in place gives the same bits as out of place
    U, M = random_site(d, r, seed=5)
    site = gpu_site(U, M)
    rsq.rsq_subspace_correct(hd, out, site, r)
    rsq.rsq_subspace_correct(hd, hd, site, r)
    torch.cuda.synchronize()
    assert torch.equal(out, hd)


def test_correct_strided_rows_and_empty_batch():
    rsq = lib()
    import torch
    d, r, n = 256, 8, 9
    U, M = random_site(d, r, seed=6)
    site = gpu_site(U, M)
    h = residual(n, d, "bf16", seed=7)
    big = torch.zeros((n, d + 64), dtype=torch.bfloat16, device="cuda")
    big[:, :d] = to_dev(h, "bf16")
    view = big[:, :d]
    outbig = torch.full((n, d + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    rsq.rsq_subspace_correct(view, outbig[:, :d], site, r)
    torch.cuda.synchronize()
    ref = online.correct(h, U, M, "bf16")
    assert rel_l2(to_host(outbig[:, :d]), ref) < 2e-2
    assert rel_l2(to_host(outbig[:, :d]), ref) <= 2 * bf16_rounding_error(h, U, M)
    assert torch.all(outbig[:, d:] == 3.0)          # padding untouched
    empty = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    rsq.rsq_subspace_correct(empty, empty, site, r)  # n = 0 enqueues nothing


QUANT_CASES = [  # dtype, n, k, bits, norm, weighted
    ("bf16", 7, 4096, 4, True, False), ("bf16", 64, 4096, 3, True, False), ("f32", 16, 256, 4, True, False),
    ("bf16", 5, 11008, 4, False, False), ("bf16", 3, 14336, 3, False, False), ("f32", 9, 96, 3, True, True),
    ("bf16", 33, 1024, 4, True, True), ("bf16", 2, 28672, 4, False, False), ("f32", 130, 32, 4, False, False),
    # the longest rows the kernel takes (four waves of 16 chunks per lane)
    ("bf16", 3, 32768, 4, True, True), ("f32", 4, 32768, 3, True, False),
]


@pytest.mark.parametrize("dtype,n,k,bits,norm,weighted", QUANT_CASES)
def test_quant_act_matches_oracle(dtype, n, k, bits, norm, weighted):
    rsq = lib()
    import torch
    print(f"case quant dtype={dtype} n={n} k={k} bits={bits} norm={norm} w={weighted}", flush=True)
    x = residual(n, k, dtype, seed=k + n, outliers=5, scale=30.0)
    if n > 2:
        x[1] = 0.0                                   # an all-zero row
    w = np.random.default_rng(1).uniform(0.5, 1.5, k).astype(np.float32) if weighted else None
    codes = empty_u8(n, rsq.rsq_packed_row_bytes(k, bits))
    scales = empty_f32(n)
    rsq.rsq_quant_act(to_dev(x, dtype), codes, scales, bits, rmsnorm=norm,
                      norm_w=None if w is None else to_dev(w, "f32"), eps=1e-5)
    torch.cuda.synchronize()
    q_ref, s_ref = online.quant_act(x, bits, norm, 1e-5, w)
    q_gpu = packing.unpack(codes.cpu().numpy(), k, bits)
    s_gpu = scales.cpu().numpy()
    ok, nbad, dmax, nontie = code_mismatch_ok(q_gpu, q_ref, quant_input(x, norm, 1e-5, w), s_gpu)
    print(f"  code mismatches={nbad} (not at a tie: {nontie}) max_level_diff={dmax}; scale max rel={np.max(np.abs(s_gpu - s_ref) / np.maximum(s_ref, 1e-30)):.2e}")
    assert ok
    assert np.all(np.abs(s_gpu - s_ref) <= 1e-6 * np.abs(s_ref))
    if n > 2:
        assert s_gpu[1] == 0 and not q_gpu[1].any()


def test_fused_correct_quant_equals_unfused_and_oracle():
    rsq = lib()
    import torch
    # the last two: the widest residual at the largest rank (32 chunks per wave, two rank blocks) on
    # the full-block path, and the widest float32 residual at the largest rank
    for dtype, d, r, n, bits in [("bf16", 1024, 32, 45, 4), ("bf16", 512, 16, 8, 3), ("f32", 256, 8, 16, 4),
                                 ("bf16", 8192, 64, 300, 4), ("f32", 4096, 64, 200, 3)]:
        print(f"case fused dtype={dtype} d={d} r={r} n={n} bits={bits}", flush=True)
        U, M = random_site(d, r, seed=11)
        site = gpu_site(U, M)
        h = residual(n, d, dtype, seed=12)
        hd = to_dev(h, dtype)
        rb = rsq.rsq_packed_row_bytes(d, bits)
        h1, c1, s1 = torch.empty_like(hd), empty_u8(n, rb), empty_f32(n)
        rsq.rsq_correct_quant(hd, h1, site, r, c1, s1, bits)
        h2, c2, s2 = torch.empty_like(hd), empty_u8(n, rb), empty_f32(n)
        rsq.rsq_subspace_correct(hd, h2, site, r)
        rsq.rsq_quant_act(h2, c2, s2, bits, rmsnorm=True)
        torch.cuda.synchronize()
        # h' bit-identical; the statistics differ only in summation order
        assert torch.equal(h1, h2)
        s1h, s2h = s1.cpu().numpy(), s2.cpu().numpy()
        assert np.all(np.abs(s1h - s2h) <= 4e-7 * s2h)
        a1 = quant_input(to_host(h1), True, 1e-5)
        ok, nbad, _, nontie = code_mismatch_ok(packing.unpack(c1.cpu().numpy(), d, bits),
                                               packing.unpack(c2.cpu().numpy(), d, bits), a1, s1h)
        assert ok, (nbad, nontie)
        # against the oracle: h' within tolerance, codes from the oracle quantiser on the GPU's h'
        err = rel_l2(to_host(h1), online.correct(h, U, M, dtype))
        assert err <= (1e-3 if dtype == "f32" else 2e-2)
        if dtype == "bf16":
            assert err <= 2 * bf16_rounding_error(h, U, M)
        q_ref, s_ref = online.quant_act(to_host(h1), bits, True, 1e-5)
        ok, nbad, _, nontie = code_mismatch_ok(packing.unpack(c1.cpu().numpy(), d, bits), q_ref, a1, s1h)
        assert ok, (nbad, nontie)
        assert np.all(np.abs(s1.cpu().numpy() - s_ref) <= 1e-6 * s_ref)


GEMM_CASES = [  # bits, n, N, K, y dtype
    (4, 1, 32, 32, "f32"), (4, 5, 96, 96, "bf16"), (3, 7, 64, 224, "f32"), (4, 64, 256, 256, "bf16"),
    (3, 65, 288, 4096, "bf16"), (4, 130, 256, 4096, "f32"), (4, 33, 512, 11008, "bf16"), (3, 200, 160, 1056, "f32"),
    (4, 300, 4096, 512, "bf16"), (4, 20, 16448, 256, "bf16"), (3, 50, 8224, 224, "f32"),
    # 16-channel decode kernel: one token block of a wide layer, int3 with a long k, three token blocks
    (4, 16, 22016, 4096, "bf16"), (3, 12, 4096, 11008, "bf16"), (4, 40, 2048, 4128, "f32"),
    # long k with the 3-step register ring (1 and 16 tokens, ragged last k step)
    (4, 1, 64, 8224, "f32"), (3, 16, 128, 16416, "bf16"),
    # int4 packed in LDS on the decode-size tiles: 64 x 64 (50 tokens) and 32 x 32 (27 tokens),
    # ragged channels and a partial 256-code k step
    (4, 50, 8224, 4128, "bf16"), (4, 27, 16448, 1056, "f32"),
    # 32-channel decode kernel in one round of workgroups: one and two 32-token fragments
    (4, 24, 6144, 4096, "bf16"), (3, 40, 8192, 1056, "f32"),
]


def _random_codes(rows, k, bits, rng, extremes=True):
    qm = packing.qmax(bits)
    q = rng.integers(-qm, qm + 1, (rows, k))
    if extremes and rows > 0:
        q[0, : min(k, 64)] = -qm
    return q


@pytest.mark.parametrize("bits,n,N,K,ydt", GEMM_CASES)
def test_qgemm_bit_exact(bits, n, N, K, ydt):
    rsq = lib()
    import torch
    print(f"case qgemm bits={bits} n={n} N={N} K={K} y={ydt}", flush=True)
    rng = np.random.default_rng(n * 7 + N + K)
    qa, qw = _random_codes(n, K, bits, rng), _random_codes(N, K, bits, rng)
    sa = rng.uniform(0.01, 2.0, n).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    a_dev = torch.from_numpy(packing.pack(qa, bits)).cuda()
    w_dev = torch.from_numpy(packing.pack(qw, bits)).cuda()
    y = torch.empty((n, N), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32, device="cuda")
    acc = torch.empty((n, N), dtype=torch.int32, device="cuda")
    rsq.rsq_qgemm(a_dev, to_dev(sa, "f32"), n, w_dev, to_dev(sw, "f32"), N, K, bits, y, acc_out=acc)
    torch.cuda.synchronize()
    acc_ref = online.gemm(qa, qw)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    y_ref = online.dequant(acc_ref, sa, sw, ydt)
    assert np.array_equal(to_host(y).astype(np.float64), np.asarray(y_ref, np.float64))
    # a second run gives the same bits (no order-dependent reductions)
    y2 = torch.empty_like(y)
    rsq.rsq_qgemm(a_dev, to_dev(sa, "f32"), n, w_dev, to_dev(sw, "f32"), N, K, bits, y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("bits,n,N,K,ydt", [(4, 40, 64, 65536, "f32"), (3, 300, 256, 65536, "bf16"),
                                             (4, 300, 96, 65536, "bf16")])
def test_qgemm_longest_k_with_extreme_accumulators(bits, n, N, K, ydt):
    """K at its limit, with rows of -qmax against rows of -qmax and +qmax.

    Accumulator 0,0 is K qmax^2 and 0,1 is -K qmax^2, the largest magnitudes
    the codes allow (the widened products then sum to 256 or 1024 times that,
    still inside int32); the decode kernel takes 40 tokens, the tiles 300.
    """
    rsq = lib()
    import torch
    print(f"case qgemm longest k bits={bits} n={n} N={N} K={K} y={ydt}", flush=True)
    rng = np.random.default_rng(K + n)
    qm = packing.qmax(bits)
    qa, qw = _random_codes(n, K, bits, rng, extremes=False), _random_codes(N, K, bits, rng, extremes=False)
    qa[0] = -qm
    qw[0] = -qm
    qw[1] = qm
    sa = rng.uniform(0.01, 2.0, n).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    y = torch.empty((n, N), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32, device="cuda")
    acc = torch.empty((n, N), dtype=torch.int32, device="cuda")
    rsq.rsq_qgemm(torch.from_numpy(packing.pack(qa, bits)).cuda(), to_dev(sa, "f32"), n,
                  torch.from_numpy(packing.pack(qw, bits)).cuda(), to_dev(sw, "f32"), N, K, bits, y, acc_out=acc)
    torch.cuda.synchronize()
    acc_ref = online.gemm(qa, qw)
    assert acc_ref[0, 0] == K * qm * qm and acc_ref[0, 1] == -K * qm * qm
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    assert np.array_equal(to_host(y).astype(np.float64), np.asarray(online.dequant(acc_ref, sa, sw, ydt), np.float64))


@pytest.mark.parametrize("bits,n,N,K", [(4, 1000, 12320, 4096), (4, 2000, 22048, 1056), (3, 2000, 22048, 4096),
                                         (4, 1800, 12224, 4096), (3, 1800, 12224, 1056),
                                         # 256 x 128 tiles (int4 packed in LDS, 256-code k steps; int3 widened)
                                         (4, 1900, 4064, 4128), (4, 2048, 4096, 11008), (3, 1900, 4064, 4128)])
def test_qgemm_large_tiles_with_ragged_edges(bits, n, N, K):
    """Shapes that take the 256 x 256, 256 x 192 or 256 x 128 tiles, with partial tiles in tokens, channels and k.

    The y-only launch (LDS-staged epilogue) must equal the launch that also
    writes the accumulators (direct epilogue); sampled blocks match the oracle.
    """
    rsq = lib()
    import torch
    print(f"case qgemm-large bits={bits} n={n} N={N} K={K}", flush=True)
    rng = np.random.default_rng(n + N + K + bits)
    qa, qw = _random_codes(n, K, bits, rng), _random_codes(N, K, bits, rng)
    sa = rng.uniform(0.01, 2.0, n).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    a_dev = torch.from_numpy(packing.pack(qa, bits)).cuda()
    w_dev = torch.from_numpy(packing.pack(qw, bits)).cuda()
    y = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
    rsq.rsq_qgemm(a_dev, to_dev(sa, "f32"), n, w_dev, to_dev(sw, "f32"), N, K, bits, y)
    y2 = torch.empty_like(y)
    acc = torch.empty((n, N), dtype=torch.int32, device="cuda")
    rsq.rsq_qgemm(a_dev, to_dev(sa, "f32"), n, w_dev, to_dev(sw, "f32"), N, K, bits, y2, acc_out=acc)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows = np.unique(np.r_[0, 255, 256, n - 1, rng.choice(n, 40, replace=False)])
    cols = np.unique(np.r_[0, 127, 128, 191, 192, 255, 256, N - 33, N - 1, rng.choice(N, 120, replace=False)])
    acc_ref = online.gemm(qa[rows], qw[cols])
    acc_gpu = acc[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.int64)
    assert np.array_equal(acc_gpu, acc_ref)
    y_gpu = to_host(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    assert np.array_equal(np.asarray(y_gpu, np.float64), np.asarray(online.dequant(acc_ref, sa[rows], sw[cols], "bf16"), np.float64))


@pytest.mark.parametrize("bits,n,N,K,ydt,inplace", [
    (4, 37, 96, 256, "bf16", False), (4, 300, 4096, 512, "bf16", True), (3, 70, 288, 1056, "f32", False),
    (4, 1000, 12320, 1024, "bf16", True), (4, 5, 64, 64, "f32", True),
])
def test_qgemm_residual_matches_oracle(bits, n, N, K, ydt, inplace):
    rsq = lib()
    import torch
    print(f"case qgemm-residual bits={bits} n={n} N={N} K={K} y={ydt} inplace={inplace}", flush=True)
    rng = np.random.default_rng(n + N + K + 11)
    qa, qw = _random_codes(n, K, bits, rng), _random_codes(N, K, bits, rng)
    sa = rng.uniform(0.01, 2.0, n).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    res = (rng.standard_normal((n, N)) * 3).astype(np.float32)
    if ydt == "bf16":
        res = round_to_bf16(res).astype(np.float32)
    res_dev = to_dev(res, ydt)
    a_dev = torch.from_numpy(packing.pack(qa, bits)).cuda()
    w_dev = torch.from_numpy(packing.pack(qw, bits)).cuda()
    y = res_dev if inplace else torch.empty_like(res_dev)
    rsq.rsq_qgemm_residual(a_dev, to_dev(sa, "f32"), n, w_dev, to_dev(sw, "f32"), N, K, bits, res_dev, y)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, n - 1, rng.choice(n, min(n, 48), replace=False)])
    acc_ref = online.gemm(qa[rows], qw)
    y_ref = online.dequant_add(acc_ref, sa[rows], sw, res[rows], ydt)
    got = to_host(y[torch.from_numpy(rows).cuda()])
    assert np.array_equal(np.asarray(got, np.float64), np.asarray(y_ref, np.float64))


@pytest.mark.parametrize("rows,k", [(1, 32), (7, 224), (300, 4096), (3, 65536)])
def test_codes_to_fp4_matches_oracle(rows, k):
    """int3 rows -> fp4 rows, byte for byte the oracle's fp4 packing of the same codes."""
    rsq = lib()
    import torch
    print(f"case codes_to_fp4 rows={rows} k={k}", flush=True)
    codes = _random_codes(rows, k, 3, np.random.default_rng(rows + k))
    out = torch.full((rows, k // 2), 0x5A, dtype=torch.uint8, device="cuda")
    rsq.rsq_codes_to_fp4(torch.from_numpy(packing.pack(codes, 3)).cuda(), rows, k, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), packing.pack_fp4(codes))


@pytest.mark.parametrize("entry,dtype,n,d", [("quant", "bf16", 33, 4096), ("quant", "f32", 5, 11008),
                                             ("quant_w", "bf16", 300, 1024), ("correct", "bf16", 2048, 4096),
                                             ("correct", "bf16", 64, 4096), ("correct_w", "f32", 40, 1024),
                                             ("fused", "bf16", 300, 4096)])
def test_fp4_codes_written_by_the_quantisers(entry, dtype, n, d):
    """bits = 3 | RSQ_FP4: the same codes as bits = 3 in the fp4 layout (and the same scales,
    h_out and y), at prefill and decode sizes (the latter through the column-split correction)."""
    rsq = lib()
    import torch
    print(f"case fp4 codes {entry} dtype={dtype} n={n} d={d}", flush=True)
    fp4 = 3 | rsq.RSQ_FP4
    assert rsq.rsq_packed_row_bytes(d, fp4) == d // 2
    x = residual(n, d, dtype, seed=n + d)
    if n > 2:
        x[1] = 0.0
    xd = to_dev(x, dtype)
    w = to_dev(np.random.default_rng(3).uniform(0.5, 1.5, d).astype(np.float32), "f32") if entry.endswith("_w") else None
    outs = {}
    for bits in (3, fp4):
        codes, scales = empty_u8(n, rsq.rsq_packed_row_bytes(d, bits)), empty_f32(n)
        h_out = y = None
        if entry.startswith("quant"):
            rsq.rsq_quant_act(xd, codes, scales, bits, rmsnorm=True, norm_w=w, eps=1e-5)
        else:
            r = 32
            U, M = subspace_site(d, r, seed=d) if d > 1024 else random_site(d, r, seed=d)
            site = gpu_site(U, M)
            h_out = torch.empty_like(xd)
            if entry.startswith("correct"):
                rsq.rsq_correct_quant(xd, h_out, site, r, codes, scales, bits, norm_w=w, eps=1e-5)
            else:
                N = 256
                qw = np.random.default_rng(9).integers(-3, 4, (N, d))
                wc = packing.pack(qw, 3) if bits == 3 else packing.pack_fp4(qw)
                sw = to_dev(np.random.default_rng(10).uniform(1e-3, 1e-2, N).astype(np.float32), "f32")
                y = torch.empty((n, N), dtype=xd.dtype, device="cuda")
                rsq.rsq_layer_fused(xd, h_out, site, r, codes, scales, torch.from_numpy(wc).cuda(), sw, N, y, bits)
        torch.cuda.synchronize()
        outs[bits] = (codes.cpu().numpy(), scales.cpu().numpy(), h_out, y)
    c3, s3, h3, y3 = outs[3]
    c4, s4, h4, y4 = outs[fp4]
    assert np.array_equal(c4, packing.pack_fp4(packing.unpack(c3, d, 3)))
    assert np.array_equal(s4, s3)
    if h3 is not None:
        assert torch.equal(h4, h3)
    if y3 is not None:
        assert torch.equal(y4, y3)


FP4_GEMM_CASES = [  # n, N, K, y dtype, residual ("none", "separate", "inplace")
    (1, 32, 32, "f32", "none"), (20, 96, 224, "bf16", "none"), (64, 256, 4096, "bf16", "separate"),
    (65, 288, 4096, "bf16", "none"), (200, 160, 1056, "f32", "none"), (300, 4096, 512, "bf16", "separate"),
    (130, 256, 4096, "f32", "inplace"), (300, 256, 65536, "bf16", "none"),
    # 256-token tiles: 256 x 256 (ragged in tokens, channels and k) and 256 x 192
    (2000, 22048, 1056, "bf16", "none"), (1800, 12224, 4096, "bf16", "inplace"),
]


@pytest.mark.parametrize("n,N,K,ydt,resmode", FP4_GEMM_CASES)
def test_qgemm_fp4_bit_exact(n, N, K, ydt, resmode):
    """The fp4 linear equals the oracle's integer GEMM and dequantisation, and the int3 kernels' output."""
    rsq = lib()
    import torch
    print(f"case qgemm_fp4 n={n} N={N} K={K} y={ydt} residual={resmode}", flush=True)
    rng = np.random.default_rng(3 * n + N + K)
    qa, qw = _random_codes(n, K, 3, rng), _random_codes(N, K, 3, rng)
    if K == 65536:                        # the largest sums the codes allow, both signs
        qa[0], qw[0], qw[1] = -3, -3, 3
    sa = rng.uniform(0.01, 2.0, n).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    tdt = torch.bfloat16 if ydt == "bf16" else torch.float32
    a3 = torch.from_numpy(packing.pack(qa, 3)).cuda()
    w3 = torch.from_numpy(packing.pack(qw, 3)).cuda()
    a4 = torch.empty((n, K // 2), dtype=torch.uint8, device="cuda")
    w4 = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    rsq.rsq_codes_to_fp4(a3, n, K, a4)
    rsq.rsq_codes_to_fp4(w3, N, K, w4)
    sa_d, sw_d = to_dev(sa, "f32"), to_dev(sw, "f32")
    res = None
    if resmode != "none":
        res = (rng.standard_normal((n, N)) * 3).astype(np.float32)
        if ydt == "bf16":
            res = round_to_bf16(res).astype(np.float32)
    if resmode == "inplace":
        y = to_dev(res, ydt)
        rsq.rsq_qgemm_fp4(a4, sa_d, n, w4, sw_d, N, K, y, residual=y)
    elif resmode == "separate":
        r_dev = to_dev(res, ydt)
        y = torch.empty((n, N), dtype=tdt, device="cuda")
        rsq.rsq_qgemm_fp4(a4, sa_d, n, w4, sw_d, N, K, y, residual=r_dev)
    else:
        y = torch.empty((n, N), dtype=tdt, device="cuda")
        acc = torch.empty((n, N), dtype=torch.int32, device="cuda")
        rsq.rsq_qgemm_fp4(a4, sa_d, n, w4, sw_d, N, K, y, acc_out=acc)
    torch.cuda.synchronize()
    rows = np.arange(n) if n * N <= 4_000_000 else np.unique(np.r_[0, n - 1, rng.choice(n, 48, replace=False)])
    acc_ref = online.gemm(qa[rows], qw)
    if resmode == "none":
        assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), acc_ref)
        y_ref = online.dequant(acc_ref, sa[rows], sw, ydt)
    else:
        y_ref = online.dequant_add(acc_ref, sa[rows], sw, res[rows], ydt)
    got = to_host(y[torch.from_numpy(rows).cuda()])
    assert np.array_equal(np.asarray(got, np.float64), np.asarray(y_ref, np.float64))
    if resmode == "none":
        # the int3 kernels on the same codes give the same bits
        y3 = torch.empty_like(y)
        rsq.rsq_qgemm(a3, sa_d, n, w3, sw_d, N, K, 3, y3)
        torch.cuda.synchronize()
        assert torch.equal(y, y3)


def test_qgemm_strided_output_and_minimum_codes():
    rsq = lib()
    import torch
    n, N, K, bits = 40, 96, 128, 4
    # -8 is outside the quantiser's range but inside the int4 format: the kernel must still be exact
    qa = np.full((n, K), -8)
    qw = np.full((N, K), -8)
    sa = np.ones(n, np.float32)
    sw = np.ones(N, np.float32)
    y = torch.full((n, N + 32), -1.0, dtype=torch.float32, device="cuda")
    acc = torch.empty((n, N), dtype=torch.int32, device="cuda")
    rsq.rsq_qgemm(torch.from_numpy(packing.pack(qa, bits)).cuda(), to_dev(sa, "f32"), n,
                  torch.from_numpy(packing.pack(qw, bits)).cuda(), to_dev(sw, "f32"), N, K, bits, y[:, :N], acc_out=acc)
    torch.cuda.synchronize()
    assert torch.all(acc == 64 * K)
    assert torch.all(y[:, :N] == float(64 * K)) and torch.all(y[:, N:] == -1.0)


@pytest.mark.parametrize("dtype,d,r,n,N,bits,in_place", [
    ("f32", 256, 8, 16, 256, 4, False), ("bf16", 4096, 32, 300, 4096, 3, False),
    # decode sizes: the column-split site and the 16-channel GEMM; in place, the full-block site
    ("bf16", 4096, 32, 1, 12288, 4, False), ("bf16", 4096, 32, 8, 4096, 3, False), ("bf16", 4096, 32, 8, 4096, 4, True)])
def test_layer_fused_matches_oracle(dtype, d, r, n, N, bits, in_place):
    """One site and its linear in one call (the second case takes the prefill tiles and int3 codes)."""
    rsq = lib()
    import torch
    print(f"case layer_fused dtype={dtype} d={d} r={r} n={n} N={N} bits={bits} in_place={in_place}", flush=True)
    U, M = random_site(d, r, seed=21) if d <= 1024 else subspace_site(d, r, seed=21)
    site = gpu_site(U, M)
    h = residual(n, d, dtype, seed=22)
    w = (np.random.default_rng(23).standard_normal((N, d)) * 0.02).astype(np.float32)
    qw, sw = prep.quantize_weight(w, bits)
    wp = packing.pack(qw, bits)
    hd = to_dev(h, dtype)
    rb = rsq.rsq_packed_row_bytes(d, bits)
    h_out, codes, scales = (hd if in_place else torch.empty_like(hd)), empty_u8(n, rb), empty_f32(n)
    y = torch.empty((n, N), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    rsq.rsq_layer_fused(hd, h_out, site, r, codes, scales, torch.from_numpy(wp).cuda(), to_dev(sw, "f32"), N, y, bits)
    torch.cuda.synchronize()
    ref = online.layer_fused(h, U, M, dtype, bits, 1e-5, wp, sw, dtype)
    assert rel_l2(to_host(h_out), ref["h_out"]) < (1e-5 if dtype == "f32" else 2e-2)
    if dtype == "bf16":
        assert rel_l2(to_host(h_out), ref["h_out"]) <= 2 * bf16_rounding_error(h, U, M)
    # downstream stages on the GPU's own h': codes, scales and y must then agree exactly
    q_ref, s_ref = online.quant_act(to_host(h_out), bits, True, 1e-5)
    q_gpu = packing.unpack(codes.cpu().numpy(), d, bits)
    s_gpu = scales.cpu().numpy()
    assert code_mismatch_ok(q_gpu, q_ref, quant_input(to_host(h_out), True, 1e-5), s_gpu)[0]
    assert np.all(np.abs(s_gpu - s_ref) <= 1e-6 * s_ref)
    y_ref = online.dequant(online.gemm(q_gpu, qw), s_gpu, sw, dtype)
    assert np.array_equal(np.asarray(to_host(y), np.float64), np.asarray(y_ref, np.float64))
    assert rel_l2(to_host(y), ref["y"]) < (1e-2 if dtype == "f32" else 3e-2)


def test_many_blocks_norm_weight_and_determinism():
    """Several waves of workgroups over the chip, a ragged last block, a norm weight, repeat runs."""
    rsq = lib()
    import torch
    d, r, bits = 8192, 32, 4
    n = 16 * 256 * 3 + 37            # more token blocks than compute units, ragged tail
    U, M = subspace_site(d, r, seed=31)
    site = gpu_site(U, M)
    h = residual(n, d, "bf16", seed=32)
    w = np.random.default_rng(33).uniform(0.5, 1.5, d).astype(np.float32)
    hd = to_dev(h, "bf16")
    outs = []
    for _ in range(2):
        h1, c1, s1 = torch.empty_like(hd), empty_u8(n, d // 2), empty_f32(n)
        rsq.rsq_correct_quant(hd, h1, site, r, c1, s1, bits, norm_w=to_dev(w, "f32"))
        outs.append((h1, c1, s1))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))
    h1, c1, s1 = outs[0]
    err = rel_l2(to_host(h1), online.correct(h, U, M, "bf16"))
    assert err < 2e-2 and err <= 2 * bf16_rounding_error(h, U, M)
    q_ref, s_ref = online.quant_act(to_host(h1), bits, True, 1e-5, w)
    assert code_mismatch_ok(packing.unpack(c1.cpu().numpy(), d, bits), q_ref,
                            quant_input(to_host(h1), True, 1e-5, w), s1.cpu().numpy())[0]
    assert np.all(np.abs(s1.cpu().numpy() - s_ref) <= 1e-6 * s_ref)



SMALL_SITE_CASES = [  # dtype, d, r, n, bits, weighted: batches small enough for the column-split site
    ("bf16", 4096, 32, 1, 4, False), ("bf16", 4096, 32, 8, 3, True), ("bf16", 4096, 32, 64, 4, False),
    ("bf16", 4096, 32, 17, 3 | 0x100, False), ("bf16", 8192, 32, 5, 4, True), ("f32", 1024, 16, 9, 4, False),
    ("bf16", 2048, 64, 24, 3, False),
]


@pytest.mark.parametrize("dtype,d,r,n,bits,weighted", SMALL_SITE_CASES)
def test_small_batch_site_matches_oracle_and_the_two_step_form(dtype, d, r, n, bits, weighted):
    """A few tokens: the column-split correction (workgroups split the columns
    of each token block), then the standalone quantiser on the stored rows. h'
    equals the correction alone bit for bit; codes and scales match the oracle
    quantiser on the GPU's own h'; a second call repeats the first exactly."""
    rsq = lib()
    import torch
    print(f"case small site dtype={dtype} d={d} r={r} n={n} bits={bits} w={weighted}", flush=True)
    assert rsq.rsq_correct_workspace_bytes(n, d) == 0
    U, M = random_site(d, r, seed=d + n) if d <= 2048 else subspace_site(d, r, seed=d + n)
    site = gpu_site(U, M)
    h = residual(n, d, dtype, seed=n + 5)
    w = np.random.default_rng(n).uniform(0.5, 1.5, d).astype(np.float32) if weighted else None
    wd = None if w is None else to_dev(w, "f32")
    hd = to_dev(h, dtype)
    rb = rsq.rsq_packed_row_bytes(d, bits)
    outs = []
    for _ in range(2):
        h1, c1, s1 = torch.empty_like(hd), empty_u8(n, rb), empty_f32(n)
        rsq.rsq_correct_quant(hd, h1, site, r, c1, s1, bits, norm_w=wd)
        outs.append((h1, c1, s1))
    h2 = torch.empty_like(hd)
    rsq.rsq_subspace_correct(hd, h2, site, r)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))
    h1, c1, s1 = outs[0]
    assert torch.equal(h1, h2)
    hp = to_host(h1)
    err = rel_l2(hp, online.correct(h, U, M, dtype))
    assert err <= (1e-5 if dtype == "f32" else 2 * bf16_rounding_error(h, U, M))
    code_bits = 3 if bits != 4 else 4
    q_ref, s_ref = online.quant_act(hp, code_bits, True, 1e-5, w)
    if bits == (3 | 0x100):
        q_gpu = packing.unpack_fp4(c1.cpu().numpy(), d)
    else:
        q_gpu = packing.unpack(c1.cpu().numpy(), d, bits)
    s_gpu = s1.cpu().numpy()
    ok, nbad, _, nontie = code_mismatch_ok(q_gpu, q_ref, quant_input(hp, True, 1e-5, w), s_gpu)
    print(f"  rel_l2={err:.2e} tie codes={nbad} not at a tie={nontie}", flush=True)
    assert ok
    assert np.all(np.abs(s_gpu - s_ref) <= 1e-6 * s_ref)
