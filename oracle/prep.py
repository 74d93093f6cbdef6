"""Offline steps of ReSpinQuant in float64 (oracle side).

Rotations. Each residual segment has its own learned D x D rotation; learning
starts at a normalised Hadamard matrix and uses a Cayley optimiser, and the
learned rotations stay close to that start (zh §2.1; it §2C; es §2A). With no
trained weights here, a learned rotation is stood in for by R = H C(eps A):
H the Sylvester-Hadamard matrix, C the Cayley transform, A a random
skew-symmetric matrix.

Basis mismatch. A block whose input and output rotations differ needs
T = R_out^T R_in at its residual junction; a single global rotation gives
T = I (zh §2.1-§2.2; nl §2B; es §2B; fr §2B. The it page writes
R_out R_in^T instead; the four others agree on R_out^T R_in).

Subspace. dT = T - I is decomposed by SVD and its top-r singular vectors form
the basis U_r of the correction subspace (it §2C; nl §2C; es §2B; fr §2C).
Inside it a dense r x r transform acts, applied as M = R_sub - I_r
(zh §2.2 step 2). The pages learn R_sub; here it takes the closed form
Q_r = U_r^T T U_r, the compression of T onto the subspace.

Weights. The rotations are fused into the weights offline (zh §2.2, offline
weight fusion, e.g. W~ = R^T W R; fr §2A, W~ = W R): for a row h in a basis
rotated by R (h~ = h R) a linear y = h W^T equals y = h~ (W R)^T, and an
output kept in a basis R' is y R' = h~ (R'^T W R)^T. Then per-output-channel
symmetric absmax quantisation with round-to-nearest (the pages name only
W4/W3; same rule as the activations).
"""
from __future__ import annotations

import numpy as np

from . import online


def hadamard(d: int) -> np.ndarray:
    """Normalised Sylvester-Hadamard matrix of order d (d a power of two): H H^T = I."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def cayley(s: np.ndarray) -> np.ndarray:
    """Cayley transform C(S) = (I - S)^-1 (I + S) of a skew-symmetric S (orthogonal, det +1)."""
    eye = np.eye(s.shape[0])
    return np.linalg.solve(eye - s, eye + s)


def rotation(a: np.ndarray, eps: float) -> np.ndarray:
    """Stand-in for a learned rotation: R = H C(eps A)."""
    return hadamard(a.shape[0]) @ cayley(eps * a)


def basis_mismatch(r_in: np.ndarray, r_out: np.ndarray) -> np.ndarray:
    """T = R_out^T R_in."""
    return r_out.T @ r_in


def principal_subspace(t: np.ndarray, r: int, check_gap: bool = True):
    """Top-r left singular vectors of dT = T - I, with all singular values.

    A rank that splits a pair of equal singular values leaves the subspace
    undefined, so a gap sigma_r - sigma_{r+1} > 1e-6 sigma_1 is required.
    """
    d = t.shape[0]
    if not 1 <= r <= d:
        raise ValueError("rank out of range")
    u, sigma, _ = np.linalg.svd(t - np.eye(d))
    if check_gap and r < d and not sigma[r - 1] - sigma[r] > 1e-6 * sigma[0]:
        raise ValueError(f"no singular-value gap at rank {r}")
    return u[:, :r], sigma


def subspace_transform(t: np.ndarray, u_r: np.ndarray) -> np.ndarray:
    """M = Q_r - I_r with Q_r = U_r^T T U_r."""
    q_r = u_r.T @ t @ u_r
    return q_r - np.eye(u_r.shape[1])


def approx_operator(u_r: np.ndarray, m: np.ndarray) -> np.ndarray:
    """The dense D x D operator the correction applies to a row: T_hat = I + U_r M U_r^T."""
    return np.eye(u_r.shape[0]) + u_r @ m @ u_r.T


def site(a_in: np.ndarray, a_out: np.ndarray, eps: float, r: int):
    """Everything one correction site needs, from its two skew generators.

    Returns a dict with T (float64), sigma, U_r and M in float64, and the
    float32 roundings U32, M32 that are the online path's inputs.
    """
    t = basis_mismatch(rotation(a_in, eps), rotation(a_out, eps))
    u_r, sigma = principal_subspace(t, r)
    m = subspace_transform(t, u_r)
    return {"T": t, "sigma": sigma, "U": u_r, "M": m,
            "U32": u_r.astype(np.float32), "M32": m.astype(np.float32)}


def fuse_weight(w: np.ndarray, right=None, left=None) -> np.ndarray:
    """W~ = left^T W right in float64 (an absent side is the identity), rounded once to float32.

    right: the rotation of the linear's input basis (K x K); left: the rotation of
    its output basis (N x N)."""
    f = np.asarray(w, np.float32).astype(np.float64)
    if right is not None:
        f = f @ np.asarray(right, np.float32).astype(np.float64)
    if left is not None:
        f = np.asarray(left, np.float32).astype(np.float64).T @ f
    return f.astype(np.float32)


def quantize_weight(w: np.ndarray, bits: int):
    """Per-output-channel (row) symmetric quantisation of a float32 weight: (codes, scales)."""
    return online.quantize(np.asarray(w, dtype=np.float32), bits)
