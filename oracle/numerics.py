"""Rounding helpers of the oracle: float64 -> bfloat16 / float32, nearest-even.

bfloat16 keeps 8 significant bits and float32's exponent range. Rounding is
done straight from the exact value (no double rounding through float32):
x = m * 2**e with 0.5 <= |m| < 1 (frexp), keep rint(m * 2**8) (ties to even).
Subnormal bfloat16 results are outside every workload here and are rejected.
"""
from __future__ import annotations

import numpy as np

_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_OVERFLOW = 2.0 ** 128


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each element (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    if np.any((ax != 0) & (ax < _BF16_MIN_NORMAL)) or np.any(~np.isfinite(x)):
        raise ValueError("round_to_bf16: subnormal or non-finite input")
    m, e = np.frexp(x)
    out = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    if np.any(np.abs(out) >= _BF16_OVERFLOW):
        raise ValueError("round_to_bf16: overflow")
    return out


def round_to_f32(x) -> np.ndarray:
    """Nearest float32 value (IEEE conversion, ties to even), returned as float32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to(dtype: str, x) -> np.ndarray:
    """Round to a storage type ("bf16" or "f32"); the result is float64 for bf16, float32 for f32."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(f"unknown storage type {dtype!r}")


def ulp_f32(x) -> np.ndarray:
    """Spacing of float32 at |x| (for tolerance reports)."""
    return np.spacing(np.abs(np.asarray(x, dtype=np.float32)))
