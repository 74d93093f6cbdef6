"""Packed storage of 4-bit and 3-bit signed codes, written from the bit-level definitions.

The pages fix only the bit widths (W4A4, W3A3: zh §4, fr §4); the layouts
below are this library's own and are the same for activations and weights.

int4: a row of K codes (K even) becomes K/2 bytes. Byte j holds code 2j in
      bits 0-3 and code 2j+1 in bits 4-7, each as a 4-bit two's complement.
int3: a row of K codes (K a multiple of 32) becomes 3K/8 bytes, 12 per group
      of 32 codes. Inside a group the 12 bytes are three 4-byte words w0, w1,
      w2 (word k = bytes 4k..4k+3); byte lane b of a word is its byte b. Code
      i of the group (u = its 3-bit two's complement pattern) has slot j = i//4
      and lane b = i%4 and is stored as:
        j = 0, 2, 4 : bits 5-7 of lane b of word j/2
        j = 1, 3, 5 : bits 2-4 of lane b of word (j-1)/2
        j = 6       : u bits 0-1 in bits 0-1 of lane b of w0, u bit 2 in bit 1 of lane b of w2
        j = 7       : u bits 0-1 in bits 0-1 of lane b of w1, u bit 2 in bit 0 of lane b of w2
fp4:  3-bit codes c in [-3, 3] as fp4 E2M1 values c/2 (the element format of
      the OCP Microscaling (MX) specification v1.0: 1 sign bit, 2 exponent
      bits with bias 1, 1 mantissa bit; exponent 0 is subnormal). A row of K
      codes (K a multiple of 32) becomes K/2 bytes, 16 per group of 32 codes:
      byte 4i + b (i, b < 4) holds code 8i + b in bits 4-7 and code 8i + 4 + b
      in bits 0-3 (the same codes as the int3 group's slots 2i and 2i+1).
"""
from __future__ import annotations

import numpy as np


def qmax(bits: int) -> int:
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    return (1 << (bits - 1)) - 1


def packed_row_bytes(k: int, bits: int) -> int:
    if bits == 4:
        if k % 2:
            raise ValueError("int4 rows need an even length")
        return k // 2
    if bits == 3:
        if k % 32:
            raise ValueError("int3 rows need a multiple of 32 codes")
        return 3 * k // 8
    raise ValueError("bits must be 3 or 4")


def _pattern(codes, bits):
    c = np.asarray(codes, dtype=np.int64)
    q = qmax(bits)
    if np.any(c < -(q + 1)) or np.any(c > q):
        raise ValueError("code out of range")
    return c & ((1 << bits) - 1)


def _signed(u, bits):
    u = np.asarray(u, dtype=np.int64)
    return np.where(u >= (1 << (bits - 1)), u - (1 << bits), u)


def pack(codes, bits: int) -> np.ndarray:
    """Pack a (rows, K) array of signed codes into (rows, packed_row_bytes(K, bits)) uint8."""
    codes = np.atleast_2d(codes)
    rows, k = codes.shape
    u = _pattern(codes, bits)
    out = np.zeros((rows, packed_row_bytes(k, bits)), dtype=np.int64)
    if bits == 4:
        out[:] = u[:, 0::2] | (u[:, 1::2] << 4)
        return out.astype(np.uint8)
    for i in range(32):
        j, b = divmod(i, 4)
        ui = u[:, i::32]                   # code i of every group, shape (rows, K/32)
        cols = lambda word: 12 * np.arange(k // 32) + 4 * word + b  # noqa: E731
        if j < 6:
            word, shift = j // 2, (5 if j % 2 == 0 else 2)
            out[:, cols(word)] |= ui << shift
        else:
            lo_word, hi_bit = (0, 1) if j == 6 else (1, 0)
            out[:, cols(lo_word)] |= ui & 3
            out[:, cols(2)] |= ((ui >> 2) & 1) << hi_bit
    return out.astype(np.uint8)


def unpack(packed, k: int, bits: int) -> np.ndarray:
    """Inverse of ``pack``: (rows, packed bytes) uint8 -> (rows, K) int64 codes."""
    p = np.atleast_2d(np.asarray(packed, dtype=np.int64))
    rows = p.shape[0]
    if p.shape[1] != packed_row_bytes(k, bits):
        raise ValueError("packed width does not match K")
    u = np.zeros((rows, k), dtype=np.int64)
    if bits == 4:
        u[:, 0::2] = p & 0xF
        u[:, 1::2] = (p >> 4) & 0xF
        return _signed(u, 4)
    for i in range(32):
        j, b = divmod(i, 4)
        cols = lambda word: 12 * np.arange(k // 32) + 4 * word + b  # noqa: E731
        if j < 6:
            word, shift = j // 2, (5 if j % 2 == 0 else 2)
            u[:, i::32] = (p[:, cols(word)] >> shift) & 7
        else:
            lo_word, hi_bit = (0, 1) if j == 6 else (1, 0)
            u[:, i::32] = (p[:, cols(lo_word)] & 3) | (((p[:, cols(2)] >> hi_bit) & 1) << 2)
    return _signed(u, 3)


def e2m1_value(nibble: int) -> float:
    """Value of a 4-bit E2M1 element (OCP MX v1.0): sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    if not 0 <= nibble < 16:
        raise ValueError("not a 4-bit pattern")
    sign = -1.0 if nibble & 8 else 1.0
    e, m = (nibble >> 1) & 3, nibble & 1
    if e == 0:
        return sign * (m / 2.0)              # subnormal: 2^(1-bias) * 0.m
    return sign * 2.0 ** (e - 1) * (1.0 + m / 2.0)


def _fp4_nibble(code: int) -> int:
    """The E2M1 pattern whose value is code/2 (zero as +0); found by decoding every pattern."""
    target = code / 2.0
    for nib in range(16):
        if e2m1_value(nib) == target and not (target == 0 and nib != 0):
            return nib
    raise ValueError(f"code {code} is not exact in E2M1 as code/2")


def pack_fp4(codes) -> np.ndarray:
    """Pack a (rows, K) array of 3-bit codes into (rows, K/2) uint8 fp4 rows (layout above)."""
    c = np.atleast_2d(np.asarray(codes, dtype=np.int64))
    rows, k = c.shape
    if k % 32:
        raise ValueError("fp4 rows need a multiple of 32 codes")
    if np.any(np.abs(c) > 3):
        raise ValueError("code out of range")
    table = np.array([_fp4_nibble(v) for v in range(-3, 4)], dtype=np.int64)   # code -3..3 -> pattern
    nib = table[c + 3]
    out = np.zeros((rows, k // 2), dtype=np.int64)
    for i in range(4):
        for b in range(4):
            hi, lo = nib[:, 8 * i + b::32], nib[:, 8 * i + 4 + b::32]   # (rows, K/32)
            out[:, 16 * np.arange(k // 32) + 4 * i + b] = (hi << 4) | lo
    return out.astype(np.uint8)


def unpack_fp4(packed, k: int) -> np.ndarray:
    """Inverse of ``pack_fp4``: (rows, K/2) uint8 -> (rows, K) int64 codes (2 x the E2M1 value)."""
    p = np.atleast_2d(np.asarray(packed, dtype=np.int64))
    if k % 32 or p.shape[1] != k // 2:
        raise ValueError("packed width does not match K")
    value2 = np.array([2.0 * e2m1_value(n) for n in range(16)])
    c = np.zeros((p.shape[0], k), dtype=np.float64)
    for i in range(4):
        for b in range(4):
            byte = p[:, 16 * np.arange(k // 32) + 4 * i + b]
            c[:, 8 * i + b::32] = value2[(byte >> 4) & 0xF]
            c[:, 8 * i + 4 + b::32] = value2[byte & 0xF]
    if np.any(c != np.rint(c)) or np.any(np.abs(c) > 3):
        raise ValueError("not a 3-bit code")
    return c.astype(np.int64)
