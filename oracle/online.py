"""Online steps of ReSpinQuant (oracle side), one token per row.

Correction (zh §2.2, "subspace residual rotation approximation", steps 1-3;
fr §2C): project y = Q^T x onto the r-dimensional subspace, transform it with
M, reproject and add to the residual. Written for row vectors h = x^T as
h' = h + ((h U_r) M) U_r^T, which is h T_hat with T_hat = I + U_r M U_r^T.
The arithmetic is float64; h' is then rounded once to the residual's storage
type.

The steps after it are not on the pages, which name only the bit widths
(W4A4, W3A3: zh §4; fr §4) and a standard linear layer once the rotations
are fused (zh §2.2; nl §2A). The readings taken here:
  RMSNorm of the stored h': a = (h' * inv) * w, inv = 1 / sqrt(mean(h'^2) + eps);
  per-token symmetric quantisation: s = max|a| / qmax, q = clamp(rint(a / s));
  per-channel weights with the same rule; y = (float(acc) * s_a) * s_w.
Where float arithmetic decides an integer code it is done in float32, the
precision of the online path: inv is the float32 rounding of the float64
value, and the products, the scale and the quotient a / s are float32
operations, rint rounding ties to even.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_to, round_to_bf16
from .packing import pack, qmax, unpack


# ---------------------------------------------------------------- correction
def project(h, u):
    """Step 1: p = h U_r (float64)."""
    return np.asarray(h, np.float64) @ np.asarray(u, np.float64)


def transform(p, m):
    """Step 2: c = p M (float64)."""
    return p @ np.asarray(m, np.float64)


def reproject(h, c, u):
    """Step 3: h + c U_r^T (float64, unrounded)."""
    return np.asarray(h, np.float64) + c @ np.asarray(u, np.float64).T


def correct(h, u, m, out_dtype: str):
    """h' = h + ((h U_r) M) U_r^T, rounded to ``out_dtype`` ("bf16" or "f32")."""
    return round_to(out_dtype, reproject(h, transform(project(h, u), m), u))


# ---------------------------------------------------------- norm + quantise
def rms_inv(x, eps: float):
    """Per row float32 rounding of 1 / sqrt(mean(x^2) + eps), x taken as stored."""
    x = np.asarray(x, np.float64)
    return (1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)).astype(np.float32)


def rmsnorm(x, eps: float, weight=None):
    """a = (x * inv) * w in float32; w = None means all ones."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    a = x32 * rms_inv(x, eps)[..., None]
    if weight is not None:
        a = a * np.asarray(weight, np.float32)
    return a


def quantize(a, bits: int):
    """Per-row symmetric quantisation of float32 values: (codes int64, scales float32).

    s = max|a| / qmax (float32 division); q = clamp(rint(a / s), -qmax, qmax)
    with a float32 quotient; a row of zeros gets s = 0 and codes 0.
    """
    a = np.atleast_2d(np.asarray(a, np.float32))
    qm = np.float32(qmax(bits))
    s = (np.max(np.abs(a), axis=1) / qm).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1))
    q = np.rint(a / safe[:, None])
    q = np.clip(q, -qm, qm).astype(np.int64)
    q[s == 0] = 0
    return q, s


def quant_act(x, bits: int, norm: bool, eps: float = 1e-5, weight=None):
    """Optional RMSNorm, then per-token quantisation: (codes, scales)."""
    a = rmsnorm(x, eps, weight) if norm else np.asarray(x, np.float64).astype(np.float32)
    return quantize(a, bits)


# ------------------------------------------------------------ GEMM, dequant
def gemm(qa, qw):
    """acc[t, j] = sum_k qa[t, k] qw[j, k], exact integers (int64).

    float64 products and sums of integer codes are exact while every partial
    sum stays below 2**53; here |acc| <= K * 49, checked below.
    """
    qa = np.asarray(qa, np.int64)
    qw = np.asarray(qw, np.int64)
    bound = qa.shape[1] * int(np.max(np.abs(qa), initial=0)) * int(np.max(np.abs(qw), initial=0))
    if bound >= 2 ** 53:
        raise ValueError("integer GEMM too large for exact float64 accumulation")
    return np.rint(qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def dequant(acc, s_a, s_w, out_dtype: str):
    """y = (float32(acc) * s_a[t]) * s_w[j], float32 products, then rounded to ``out_dtype``."""
    acc = np.asarray(acc, np.int64)
    if np.any(np.abs(acc) >= 2 ** 24):
        raise ValueError("accumulator not exactly representable in float32")
    y = (acc.astype(np.float32) * np.asarray(s_a, np.float32)[:, None]) * np.asarray(s_w, np.float32)[None, :]
    if out_dtype == "f32":
        return y
    return round_to_bf16(y.astype(np.float64))


def dequant_add(acc, s_a, s_w, residual, out_dtype: str):
    """y = out_dtype(v + float32(residual)) with v = (float32(acc) * s_a[t]) * s_w[j] in float32.

    The residual add of a decoder block (the junction structure: zh §2.1;
    fr §2B) taken into the linear's output, rounded once.
    """
    acc = np.asarray(acc, np.int64)
    if np.any(np.abs(acc) >= 2 ** 24):
        raise ValueError("accumulator not exactly representable in float32")
    v = (acc.astype(np.float32) * np.asarray(s_a, np.float32)[:, None]) * np.asarray(s_w, np.float32)[None, :]
    y = v + np.asarray(residual, np.float32)
    if out_dtype == "f32":
        return y
    return round_to_bf16(y.astype(np.float64))


# ------------------------------------------------ entry points on packed data
def subspace_correct(h, u, m, dtype: str):
    return correct(h, u, m, dtype)


def quant_act_packed(x, bits: int, norm: bool, eps: float = 1e-5, weight=None):
    q, s = quant_act(x, bits, norm, eps, weight)
    return pack(q, bits), s, q


def qgemm_packed(a_codes, a_scales, w_codes, w_scales, k: int, bits: int, y_dtype: str):
    qa = unpack(a_codes, k, bits)
    qw = unpack(w_codes, k, bits)
    acc = gemm(qa, qw)
    return dequant(acc, a_scales, w_scales, y_dtype), acc


def qgemm_residual_packed(a_codes, a_scales, w_codes, w_scales, k: int, bits: int, residual, y_dtype: str):
    acc = gemm(unpack(a_codes, k, bits), unpack(w_codes, k, bits))
    return dequant_add(acc, a_scales, w_scales, residual, y_dtype), acc


def layer_fused(h, u, m, h_dtype: str, bits: int, eps: float, w_codes, w_scales,
                y_dtype: str, norm_weight=None):
    """correction -> RMSNorm -> quantisation -> quantised linear, one site."""
    hp = correct(h, u, m, h_dtype)
    codes, scales, q = quant_act_packed(hp, bits, True, eps, norm_weight)
    k = np.asarray(h).shape[1]
    y, acc = qgemm_packed(codes, scales, w_codes, w_scales, k, bits, y_dtype)
    return {"h_out": hp, "codes": codes, "scales": scales, "q": q, "y": y, "acc": acc}


def layer_linear_path(h, site_a, site_b, weights, o_in, down_in, h_dtype, bits, eps, y_dtype):
    """One decoder layer's linear path (two correction sites, four quantised linears).

    site_a / site_b: (U_r, M). weights: name -> (packed codes, scales) for
    "qkv", "o", "gate_up", "down". Site B reads site A's corrected residual
    (the attention output and its residual add are not part of this path).
    """
    d = np.asarray(h).shape[1]
    out = {}
    a = layer_fused(h, *site_a, h_dtype, bits, eps, *weights["qkv"], y_dtype)
    out["siteA"], out["qkv"] = a, a["y"]
    oc, os_, _ = quant_act_packed(o_in, bits, False)
    out["o"] = qgemm_packed(oc, os_, *weights["o"], d, bits, y_dtype)[0]
    b = layer_fused(a["h_out"], *site_b, h_dtype, bits, eps, *weights["gate_up"], y_dtype)
    out["siteB"], out["gate_up"] = b, b["y"]
    f = np.asarray(down_in).shape[1]
    dc, ds, _ = quant_act_packed(down_in, bits, False)
    out["down"] = qgemm_packed(dc, ds, *weights["down"], f, bits, y_dtype)[0]
    return out


def layer_chained(h, site_a, site_b, weights, o_in, down_in, h_dtype, bits, eps, y_dtype):
    """One decoder layer with its residual stream carried through (two sites).

    h_a = correct_A(h); q|k|v from h_a; h2 = h_a + o_proj(o_in);
    h_b = correct_B(h2); gate|up from h_b; h3 = h_b + down_proj(down_in).
    The attention core and SiLU * up are stood in for by o_in and down_in;
    each residual add is rounded once to the residual's dtype. h3 is the next
    layer's input.
    """
    d = np.asarray(h).shape[1]
    out = {}
    a = layer_fused(h, *site_a, h_dtype, bits, eps, *weights["qkv"], y_dtype)
    out["siteA"], out["qkv"] = a, a["y"]
    oc, os_, _ = quant_act_packed(o_in, bits, False)
    out["h2"] = qgemm_residual_packed(oc, os_, *weights["o"], d, bits, a["h_out"], h_dtype)[0]
    b = layer_fused(out["h2"], *site_b, h_dtype, bits, eps, *weights["gate_up"], y_dtype)
    out["siteB"], out["gate_up"] = b, b["y"]
    f = np.asarray(down_in).shape[1]
    dc, ds, _ = quant_act_packed(down_in, bits, False)
    out["h3"] = qgemm_residual_packed(dc, ds, *weights["down"], f, bits, b["h_out"], h_dtype)[0]
    return out
