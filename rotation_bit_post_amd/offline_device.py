"""Offline conversion of a correction site on the device (torch, float64).

The same conversion as ``offline.convert_site`` - T = R_out^T R_in, the top-r
singular subspace of dT = T - I, M = U_r^T T U_r - I_r (ReSpinQuant zh 2.1-2.2;
it 2C; nl 2B-2C; fr 2B-2C) - run on the GPU so that preparing a model's
junctions takes a fraction of a second each instead of a host eigensolver's
tens of seconds at D = 4096.

The subspace comes from block subspace iteration on the symmetric positive
semi-definite S = dT^T dT = 2I - T - T^T (its top-r eigenvectors are dT's top-r
left and right singular vectors, dT being normal): a block of p = 2r + 8
vectors is multiplied by S and re-orthonormalised (Cholesky QR) until the
Rayleigh-Ritz residual of the top r vectors falls below the tolerance. The
iteration converges at the rate lambda_{p+1} / lambda_r per step. As on the
host, a rank that splits a pair of equal singular values (no gap at r) is
refused.
"""
from __future__ import annotations

import numpy as np


def synthetic_rotation_device(a, eps: float, device="cuda"):
    """H C(eps A) on the device in float64 (H the normalised Sylvester-Hadamard matrix)."""
    import torch
    from .offline import sylvester_hadamard
    a = torch.as_tensor(np.asarray(a), dtype=torch.float64, device=device)
    eye = torch.eye(a.shape[0], dtype=torch.float64, device=device)
    c = torch.linalg.solve(eye - eps * a, eye + eps * a)
    h = torch.as_tensor(sylvester_hadamard(a.shape[0]), dtype=torch.float64, device=device)
    return h @ c


def _cholesky_qr(y):
    import torch
    g = y.T @ y
    l = torch.linalg.cholesky(g)
    return torch.linalg.solve_triangular(l, y.T, upper=False).T  # y L^-T


def convert_site_device(r_in, r_out, r: int, tol: float = 1e-10, max_iters: int = 3000, seed: int = 0):
    """(U_r, M) in float32 numpy, plus the iteration count and final residual.

    r_in, r_out: float64 rotations (torch tensors on the device, or numpy).
    """
    import torch
    dev = r_in.device if isinstance(r_in, torch.Tensor) else torch.device("cuda")
    r_in = torch.as_tensor(r_in, dtype=torch.float64, device=dev)
    r_out = torch.as_tensor(r_out, dtype=torch.float64, device=dev)
    t = r_out.T @ r_in
    d = t.shape[0]
    if not 1 <= r <= d:
        raise ValueError("rank out of range")
    s = 2.0 * torch.eye(d, dtype=torch.float64, device=dev) - t - t.T
    s = 0.5 * (s + s.T)
    p = min(d, 2 * r + 8)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = _cholesky_qr(torch.randn(d, p, dtype=torch.float64, generator=gen).to(dev))
    res = float("inf")
    it = 0
    lam = vec = None
    while it < max_iters:
        for _ in range(10):
            q = _cholesky_qr(s @ q)
        it += 10
        # Rayleigh-Ritz on the block
        h = q.T @ (s @ q)
        lam, w = torch.linalg.eigh(0.5 * (h + h.T))
        lam, w = lam.flip(0), w.flip(1)             # descending
        vec = q @ w[:, :r]
        res = float(torch.linalg.matrix_norm(s @ vec - vec * lam[:r]) / max(float(lam[0]), 1e-300))
        if res < tol:
            break
    if r < d and not float(lam[r - 1] - lam[r]) > 1e-6 * float(lam[0]):
        raise ValueError(f"no singular-value gap at rank {r}")
    m = vec.T @ t @ vec - torch.eye(r, dtype=torch.float64, device=dev)
    return (vec.to(torch.float32).cpu().numpy(), m.to(torch.float32).cpu().numpy(), it, res)
