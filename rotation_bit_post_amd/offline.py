"""Offline conversion of one correction site (host, float64, once per model).

This is the step before the online path: from a block's input and output
rotations to the basis U_r and the subspace transform M that
``rsq_site_prepare`` lays out for the kernels. It runs once per model on the
host, like weight packing, and is not part of the per-token path.

ReSpinQuant (zh 2.1-2.2; it 2C; nl 2B-2C; fr 2B-2C): T = R_out^T R_in; the
principal subspace of dT = T - I is spanned by its top-r singular vectors;
inside it the rotation is applied as M = R_sub - I_r, here with
R_sub = U_r^T T U_r. Because T is orthogonal, dT is normal and
dT^T dT = dT dT^T = 2I - T - T^T, so its left and right top-r singular
subspaces are both the top-r eigenspace of that symmetric matrix; a partial
symmetric eigensolver finds it without a full SVD.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg as sla


def sylvester_hadamard(d: int) -> np.ndarray:
    """Normalised Walsh-Hadamard matrix, entry (i, j) = (-1)^popcount(i & j) / sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("order must be a power of two")
    idx = np.arange(d, dtype=np.uint32)
    parity = np.zeros((d, d), dtype=np.uint32)
    x = idx[:, None] & idx[None, :]
    while np.any(x):
        parity ^= x & 1
        x >>= 1
    return (1.0 - 2.0 * parity) / np.sqrt(d)


def cayley_rotation(a: np.ndarray, eps: float) -> np.ndarray:
    """(I - eps A)^-1 (I + eps A) for skew-symmetric A: orthogonal, determinant +1."""
    eye = np.eye(a.shape[0])
    return sla.solve(eye - eps * a, eye + eps * a, assume_a="gen")


def synthetic_rotation(a: np.ndarray, eps: float) -> np.ndarray:
    """Stand-in for a learned rotation near its Hadamard start: H C(eps A)."""
    return sylvester_hadamard(a.shape[0]) @ cayley_rotation(a, eps)


def mismatch(r_in: np.ndarray, r_out: np.ndarray) -> np.ndarray:
    """T = R_out^T R_in, the rotation a junction between the two bases needs."""
    return r_out.T @ r_in


def convert_site(r_in: np.ndarray, r_out: np.ndarray, r: int):
    """(U_r, M) in float32 for a junction with rotations r_in (input) and r_out (output)."""
    return convert_mismatch(mismatch(r_in, r_out), r)


def convert_mismatch(t: np.ndarray, r: int):
    """(U_r, M) in float32 from the mismatch T (float64, orthogonal)."""
    d = t.shape[0]
    if not 1 <= r <= d:
        raise ValueError("rank out of range")
    s = 2.0 * np.eye(d) - t - t.T
    s = 0.5 * (s + s.T)
    lo = max(d - r - 1, 0)
    w, v = sla.eigh(s, subset_by_index=[lo, d - 1])      # ascending; top r (+1 for the gap check)
    if r < d and not w[-r] - w[-r - 1] > 1e-6 * w[-1]:
        raise ValueError(f"no singular-value gap at rank {r}")
    u = v[:, -r:][:, ::-1]
    m = u.T @ t @ u - np.eye(r)
    return np.ascontiguousarray(u, dtype=np.float32), np.ascontiguousarray(m, dtype=np.float32)
