"""Seeded random draws. Nothing here computes any step of the method.

Every array is a pure function of (workload seed family, stream, shape):
``numpy.random.default_rng(numpy.random.SeedSequence([seed_id, stream]))``.
"""
from __future__ import annotations

import numpy as np

from .workloads import Workload, INPUT_STREAMS, LOW_RANK_STREAMS, SKEW_STREAMS, WEIGHT_STREAMS


def _rng(seed_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed_id, stream]))


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits.

    This only gives the synthetic residual its storage type; finite inputs only.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(cfg: Workload) -> np.ndarray:
    """Sorted indices of the outlier channels, drawn without replacement."""
    return np.sort(_rng(cfg.seed_id, 3).choice(cfg.D, cfg.n_outliers, replace=False))


def residual(cfg: Workload, n: int | None = None) -> np.ndarray:
    """Residual stream h, shape (n, D), float32 values in the workload's storage type.

    Standard normal entries; the outlier channels (the same for every token)
    are multiplied by ``cfg.outlier_scale``. For bf16 workloads the values are
    rounded to bfloat16 and returned as float32 holding exactly those values.
    Rows are drawn in order, so a smaller ``n`` gives the head of a larger
    draw: a decode batch is the first rows of the prefill batch of its family.
    """
    n = cfg.n if n is None else n
    h = _rng(cfg.seed_id, 0).standard_normal((n, cfg.D), dtype=np.float32)
    h[:, outlier_channels(cfg)] *= np.float32(cfg.outlier_scale)
    if cfg.h_dtype == "bf16":
        h = bf16_bits_to_f32(to_bf16_bits(h))
    return np.ascontiguousarray(h)


def skew_generator(cfg: Workload, site: str, which: str) -> np.ndarray:
    """Skew-symmetric D x D float64 matrix with independent N(0,1) off-diagonal entries.

    ``site`` is "A" (attention input) or "B" (FFN input); ``which`` is "in" or "out".
    """
    G = _rng(cfg.seed_id, SKEW_STREAMS[(site, which)]).standard_normal((cfg.D, cfg.D))
    U = np.triu(G, 1)
    return U - U.T


def low_rank_skew(cfg: Workload, site: str, which: str, k: int) -> np.ndarray:
    """Skew-symmetric D x D float64 matrix of rank 2k: (P Q^T - Q P^T) / D, P and Q independent
    D x k standard normal draws (spectral norm about 1).

    A rotation built from it differs from its start only inside a 2k-dimensional subspace, so
    the mismatch between two such rotations has rank at most 4k.
    """
    if not 1 <= 2 * k <= cfg.D:
        raise ValueError("k out of range")
    rng = _rng(cfg.seed_id, LOW_RANK_STREAMS[(site, which)])
    P = rng.standard_normal((cfg.D, k))
    Q = rng.standard_normal((cfg.D, k))
    S = P @ Q.T
    return (S - S.T) / cfg.D


def weight(cfg: Workload, name: str, rows: int, cols: int) -> np.ndarray:
    """Dense weight, shape (rows, cols), float32 N(0, sigma_w^2)."""
    z = _rng(cfg.seed_id, WEIGHT_STREAMS[name]).standard_normal((rows, cols), dtype=np.float32)
    z *= np.float32(cfg.sigma_w)
    return z


def linear_input(cfg: Workload, which: str, n: int, width: int) -> np.ndarray:
    """Stand-in input of a linear not fed by a correction site (o_proj or down_proj).

    N(0,1), no outliers, rounded to bf16 for bf16 workloads.
    """
    x = _rng(cfg.seed_id, INPUT_STREAMS[which]).standard_normal((n, width), dtype=np.float32)
    if cfg.h_dtype == "bf16":
        x = bf16_bits_to_f32(to_bf16_bits(x))
    return np.ascontiguousarray(x)
