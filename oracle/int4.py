"""Symmetric INT4 group-128 quantizer, 4-bit packing and dequant (oracle).

[GPT54-INT4] §3.2: weights are viewed in groups of 128; each group's scale is
its maximum absolute value divided by 7, and the codes are round(w / scale)
clamped to [-7, 7] and stored as int8 before packing.  The comment there speaks
of a zero point, but the code is symmetric, so there is none.

Readings where the page is silent:
* Groups are 128 consecutive k of one row of the row-major [M][K] weight.
* The scale is stored as fp16: the fp64 quotient max|w| / 7 rounded to nearest
  even.  For bf16 inputs the fp64 quotient cannot fall on an fp16 rounding
  midpoint unless it is exact, so this is the correctly rounded scale.
* Codes are taken against the stored fp16 scale with the fp64 quotient rounded
  half-to-even (exact for these operand widths); dequant is q * s.
* A group with max |w| = 0, or whose fp16 scale underflows to 0, gets s = 1.0 and
  q = 0; an fp16 overflow of the scale is an error.
* Packing (parity unpinned by the pages, fixed here): code c = q + 8 in [1, 15]
  (0 is never written); 32-bit word w of a row holds elements 8w .. 8w+7, the
  even ones in the low half and the odd ones in the high half: element 8w + t
  sits at bit 4*(t // 2) when t is even and at bit 16 + 4*(t // 2) when t is odd.
  Row words are contiguous.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_value, fp16_rne, fp16_value, FP16_ONE

GROUP = 128


def quantize(w_bits: np.ndarray):
    """w_bits uint16 [M][K] -> (q int8 [M][K], scale fp16 bits uint16 [M][K/128])."""
    M, K = w_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = bf16_value(w_bits).reshape(M, K // GROUP, GROUP)
    amax = np.abs(w).max(axis=-1)
    s_bits = fp16_rne(amax / 7.0)
    if np.any((s_bits & 0x7FFF) == 0x7C00):
        raise ValueError("int4 scale overflows fp16")
    zero = (amax == 0) | (s_bits == 0)
    s_bits = np.where(zero, FP16_ONE, s_bits).astype(np.uint16)
    s = fp16_value(s_bits)[..., None]
    q = np.clip(np.rint(w / s), -7, 7)
    q = np.where(zero[..., None], 0, q)
    return q.reshape(M, K).astype(np.int8), s_bits


# bit position of element t (0..7) inside its word: evens low half, odds high half
SHIFTS = np.array([4 * (t // 2) + (16 if t % 2 else 0) for t in range(8)], dtype=np.int64)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """q int8 [M][K] in [-7, 7] -> uint32 [M][K/8], code q+8 at SHIFTS[k % 8]."""
    M, K = q.shape
    c = (q.astype(np.int64) + 8).reshape(M, K // 8, 8)
    return (c << SHIFTS).sum(axis=-1).astype(np.uint32)


def unpack_codes(words: np.ndarray, K: int) -> np.ndarray:
    """uint32 [M][K/8] -> q int8 [M][K]; raises on the unused code 0."""
    M = words.shape[0]
    shifts = SHIFTS.astype(np.uint32)
    c = (words.astype(np.uint32)[..., None] >> shifts) & 15
    if np.any(c == 0):
        raise ValueError("invalid int4 code 0")
    return (c.astype(np.int8) - 8).reshape(M, K)


def dequant(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    M, K = q.shape
    s = fp16_value(s_bits)
    return (q.reshape(M, K // GROUP, GROUP).astype(np.float64) * s[..., None]).reshape(M, K)


def pack(w_bits: np.ndarray) -> dict:
    q, s = quantize(w_bits)
    return {"codes": pack_codes(q), "scales": s}


def unpack_dequant(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    return dequant(unpack_codes(codes, K), scales)
