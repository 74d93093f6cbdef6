"""Shared helpers of the GPU parity tests: device transfers and cached oracle sites."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import synth
from oracle import online, prep


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def lib():
    import rotation_bit_post_amd as rsq  # raises if librsq.so is missing: no fallback
    return rsq


def to_dev(x, dtype: str):
    """numpy -> device tensor; dtype "bf16" expects bf16-exact values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def empty_u8(rows, cols):
    import torch
    return torch.empty((rows, cols), dtype=torch.uint8, device="cuda")


def empty_f32(*shape):
    import torch
    return torch.empty(shape, dtype=torch.float32, device="cuda")


@functools.lru_cache(maxsize=None)
def oracle_site(wl, which: str, r: int):
    """Oracle prep of a synthetic site (float64 SVD), cached per test session."""
    cfg = synth.workload(wl)
    s = prep.site(synth.skew_generator(cfg, which, "in"), synth.skew_generator(cfg, which, "out"), cfg.eps_rot, r)
    return s["U32"], s["M32"], s["sigma"]


@functools.lru_cache(maxsize=None)
def oracle_basis_all(wl, which: str, r_max: int):
    """U (all ranks up to r_max) and T of a site: one SVD serves a rank sweep."""
    cfg = synth.workload(wl)
    t = prep.basis_mismatch(prep.rotation(synth.skew_generator(cfg, which, "in"), cfg.eps_rot),
                            prep.rotation(synth.skew_generator(cfg, which, "out"), cfg.eps_rot))
    u, sigma = prep.principal_subspace(t, r_max)
    return u, t, sigma


def site_for_rank(wl, which: str, r: int, r_max: int = 64):
    u, t, _ = oracle_basis_all(wl, which, r_max)
    ur = u[:, :r]
    m = prep.subspace_transform(t, ur)
    return ur.astype(np.float32), m.astype(np.float32)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def quant_input(x, norm: bool, eps: float = 1e-5, weight=None) -> np.ndarray:
    """The quantiser's float32 input as the oracle forms it from x as stored:
    its RMSNorm (x * inv) * w when norm is set, else x itself."""
    if norm:
        return online.rmsnorm(x, eps, weight)
    return np.asarray(x, np.float64).astype(np.float32)


def code_mismatch_ok(gpu_codes, ref_codes, a, scales, max_frac=1e-4, ulps=16):
    """Codes may differ only at rounding ties of the per-token quantiser.

    Every differing code must (1) differ by one level, (2) sit where a / s,
    taken in float64 from the float32 quantiser input a (formed from the
    GPU's own h') and the GPU's per-row scale s, lies within `ulps` float32
    ulps of a half-integer - a tie that a last-bit difference in the row's
    statistics can tip either way - and (3) the differing codes are at most
    max_frac of all. Returns (ok, differing codes, largest level difference,
    differing codes that are not at a tie).
    """
    g = np.asarray(gpu_codes, np.int64)
    r = np.asarray(ref_codes, np.int64)
    d = np.abs(g - r)
    bad = np.nonzero(d)
    nbad = int(bad[0].size)
    dmax = int(d.max(initial=0))
    if nbad == 0:
        return True, 0, 0, 0
    a64 = np.asarray(a, np.float32).astype(np.float64)
    s64 = np.asarray(scales, np.float32).astype(np.float64).reshape(-1)
    s_el = s64[bad[0]]
    pos = s_el > 0                    # a zero row has s = 0 and admits no difference
    t = a64[bad] / np.where(pos, s_el, 1.0)
    dist = np.abs(t - (np.floor(t) + 0.5))
    at_tie = pos & (dist <= ulps * float(np.finfo(np.float32).eps) * np.abs(t))
    not_tie = int(np.sum(~at_tie))
    ok = dmax <= 1 and not_tie == 0 and nbad / d.size <= max_frac
    return ok, nbad, dmax, not_tie


def bf16_rounding_error(h, U, M) -> float:
    """Relative L2 distance of the oracle's bf16 corrected residual from its own
    unrounded float64 value: the rounding the stored h' cannot avoid."""
    exact = online.reproject(h, online.transform(online.project(h, U), M), U)
    return rel_l2(online.correct(h, U, M, "bf16"), exact)


def subspace_site(d, r, seed, eps=0.3):
    """(U32, M32) with U an orthonormal d x r basis and M = Q - I for an orthogonal r x r Q.

    The correction's arithmetic needs no full-width rotation behind (U, M):
    this site is as valid an input as one from a mismatch's SVD and costs no
    d x d solve or SVD (at d = 8192 those take minutes on the host).
    """
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((d, r)))
    g = np.random.default_rng(seed + 1).standard_normal((r, r))
    a = np.triu(g, 1)
    q = prep.cayley(eps * (a - a.T))
    return u.astype(np.float32), (q - np.eye(r)).astype(np.float32)
