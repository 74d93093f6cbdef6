"""Offline conversion of a correction site with its large products on the device (torch, float64).

The same conversion as ``offline.convert_site`` - T = R_out^T R_in, the top-r
singular subspace of dT = T - I, M = U_r^T T U_r - I_r (ReSpinQuant zh 2.1-2.2;
it 2C; nl 2B-2C; fr 2B-2C) - with every D x D product on the GPU, so that
preparing a model's junctions takes about a second each instead of a host
eigensolver's tens of seconds at D = 4096.

The subspace comes from block subspace iteration on the symmetric positive
semi-definite S = dT^T dT = 2I - T - T^T (its top-r eigenvectors are dT's top-r
left and right singular vectors, dT being normal): a block of p = 4r + 16
vectors is multiplied by S and re-orthonormalised (Cholesky QR) until the
Rayleigh-Ritz residual of the top r vectors falls below the tolerance. The
iteration converges at the rate lambda_{p+1} / lambda_r per step, and the
spectrum of the synthetic mismatches is dense (at D = 8192 a block of 2r + 8
left a residual of 8e-6 after 3000 steps), hence the wide block; a site that
has not converged after max_iters steps is refused, as is a rank that splits a
pair of equal singular values (no gap at r).

Only matrix products run on the device. The Cayley transform of each rotation
is a float64 solve on the host (the same routine as the host conversion), and
the p x p factorisations of the iteration (Cholesky, triangular inverse,
symmetric eigensolver) run on the host in numpy: they are tiny, and the
device keeps no dense-solver call.
"""
from __future__ import annotations

import numpy as np


def synthetic_rotation_device(a, eps: float, device="cuda"):
    """H C(eps A) in float64 on the device: the Cayley transform solved on the host, the product with the
    normalised Sylvester-Hadamard matrix H on the device."""
    import torch
    from .offline import cayley_rotation, sylvester_hadamard
    a = np.asarray(a, np.float64)
    c = torch.as_tensor(cayley_rotation(a, eps), dtype=torch.float64, device=device)
    h = torch.as_tensor(sylvester_hadamard(a.shape[0]), dtype=torch.float64, device=device)
    return h @ c


def _cholesky_qr(y):
    """Orthonormal columns spanning y: y L^-T with L L^T = y^T y (Gram on the device, factor on the host)."""
    import torch
    g = (y.T @ y).cpu().numpy()
    l_inv_t = np.linalg.inv(np.linalg.cholesky(0.5 * (g + g.T))).T
    return y @ torch.as_tensor(l_inv_t, dtype=y.dtype, device=y.device)


def convert_site_device(r_in, r_out, r: int, tol: float = 1e-10, max_iters: int = 10000, seed: int = 0):
    """(U_r, M) in float32 numpy, plus the iteration count and final residual.

    r_in, r_out: float64 rotations (torch tensors on the device, or numpy).
    Raises ValueError if the residual is still >= tol after max_iters steps.
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
    p = min(d, 4 * r + 16)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = _cholesky_qr(torch.randn(d, p, dtype=torch.float64, generator=gen).to(dev))
    res = float("inf")
    it = 0
    lam = vec = None
    while it < max_iters:
        for _ in range(min(10, max_iters - it)):
            q = _cholesky_qr(s @ q)
            it += 1
        # Rayleigh-Ritz on the block (p x p eigenproblem on the host)
        sq = s @ q
        h = (q.T @ sq).cpu().numpy()
        lam_h, w_h = np.linalg.eigh(0.5 * (h + h.T))
        lam_h, w_h = lam_h[::-1].copy(), w_h[:, ::-1].copy()      # descending
        w = torch.as_tensor(w_h[:, :r], dtype=torch.float64, device=dev)
        vec = q @ w
        lam = lam_h
        resid = sq @ w - vec * torch.as_tensor(lam[:r], dtype=torch.float64, device=dev)
        res = float(torch.linalg.vector_norm(resid) / max(float(lam[0]), 1e-300))
        if res < tol:
            break
    if not res < tol:
        raise ValueError(f"subspace iteration did not converge: residual {res:.3e} >= {tol:.1e} after {it} steps")
    if r < d and not float(lam[r - 1] - lam[r]) > 1e-6 * float(lam[0]):
        raise ValueError(f"no singular-value gap at rank {r}")
    m = vec.T @ t @ vec - torch.eye(r, dtype=torch.float64, device=dev)
    return (vec.to(torch.float32).cpu().numpy(), m.to(torch.float32).cpu().numpy(), it, res)


def fuse_weight_device(w, right=None, left=None):
    """W~ = left^T W right on the device with the library's rotation kernel (one launch per side,
    float64 sums, one float32 rounding per side); w, right, left: float32 device tensors."""
    import torch
    from . import _binding as B
    out = w
    if right is not None:
        nxt = torch.empty_like(w)
        B.rsq_rotate_weight(out, right, B.RSQ_ROTATE_RIGHT, nxt)
        out = nxt
    if left is not None:
        nxt = torch.empty_like(w)
        B.rsq_rotate_weight(out, left, B.RSQ_ROTATE_LEFT, nxt)
        out = nxt
    return out
