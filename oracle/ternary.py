"""Block-ternary absmean quantizer, its 2-bit packing and dequant (oracle).

[Bonsai2] §1.2 defines ``block_ternary``: split the weight into blocks of 128
values, take each block's mean absolute value as its scale, and round w / scale
to the nearest integer clamped to [-1, 1].  Mean (not max) keeps one outlier from
zeroing the whole block.  [Bonsai2] §3.4 / §5.5: a block that is entirely zero
gets scale 1 and is flagged all-zero.

Readings where the page is silent (each listed in the design notes):
* W is [M][K] row-major (row = output channel), blocks are 128 consecutive k of
  one row (the page's reshape(-1, 128) on a row-major weight).
* The mean is the fp64 sum of |w| taken in index order, divided by 128.
* The page adds eps = 1e-8 to the scale only to avoid dividing by zero; the
  all-zero rule covers that case, so eps is dropped.  The scale is stored as
  fp16 (round to nearest even from the exact fp64 mean) and the codes are taken
  against that stored scale, so dequant(q, s_stored) is what a GEMV uses.
* Rounding is half-to-even (torch.round); |w| == s / 2 therefore gives 0.
* A block whose mean is 0, or whose fp16 scale underflows to 0, gets s = 1.0
  and q = 0 (the all-zero rule).  A scale that overflows fp16 is an error.
* Packing (parity unpinned by the pages, fixed here): code c = q + 1 in
  {0, 1, 2}; 32-bit word w of a row holds elements 16w .. 16w+15, the even ones
  in the low half and the odd ones in the high half: element 16w + t sits at bit
  2*(t // 2) when t is even and at bit 16 + 2*(t // 2) when t is odd.  The words
  of a row are contiguous, rows follow each other.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_value, fp16_rne, fp16_value, FP16_ONE

BLOCK = 128


def quantize(w_bits: np.ndarray):
    """w_bits uint16 [M][K] -> (q int8 [M][K], scale fp16 bits uint16 [M][K/128])."""
    M, K = w_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    w = bf16_value(w_bits).reshape(M, K // BLOCK, BLOCK)
    total = np.zeros((M, K // BLOCK))
    for i in range(BLOCK):                            # fp64, in index order
        total += np.abs(w[..., i])
    mean = total / BLOCK                              # /128 is exact
    s_bits = fp16_rne(mean)
    if np.any((s_bits & 0x7FFF) == 0x7C00):
        raise ValueError("ternary scale overflows fp16")
    zero = (mean == 0) | (s_bits == 0)
    s_bits = np.where(zero, FP16_ONE, s_bits).astype(np.uint16)
    s = fp16_value(s_bits)[..., None]
    q = np.clip(np.rint(w / s), -1, 1)
    q = np.where(zero[..., None], 0, q)
    return q.reshape(M, K).astype(np.int8), s_bits


# bit position of element t (0..15) inside its word: evens low half, odds high half
SHIFTS = np.array([2 * (t // 2) + (16 if t % 2 else 0) for t in range(16)], dtype=np.int64)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """q int8 [M][K] in {-1,0,1} -> uint32 [M][K/16], code q+1 at SHIFTS[k % 16]."""
    M, K = q.shape
    c = (q.astype(np.int64) + 1).reshape(M, K // 16, 16)
    return (c << SHIFTS).sum(axis=-1).astype(np.uint32)


def unpack_codes(words: np.ndarray, K: int) -> np.ndarray:
    """uint32 [M][K/16] -> q int8 [M][K]; raises on the unused code 3."""
    M = words.shape[0]
    shifts = SHIFTS.astype(np.uint32)
    c = (words.astype(np.uint32)[..., None] >> shifts) & 3
    if np.any(c == 3):
        raise ValueError("invalid ternary code 3")
    return (c.astype(np.int8) - 1).reshape(M, K)


def dequant(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """fp64 [M][K] = q * s (exact)."""
    M, K = q.shape
    s = fp16_value(s_bits)
    return (q.reshape(M, K // BLOCK, BLOCK).astype(np.float64) * s[..., None]).reshape(M, K)


def pack(w_bits: np.ndarray) -> dict:
    """Packed sections {'codes', 'scales'} of a bf16 weight."""
    q, s = quantize(w_bits)
    return {"codes": pack_codes(q), "scales": s}


def unpack_dequant(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Dense fp64 weight from the packed sections."""
    return dequant(unpack_codes(codes, K), scales)


def zero_fraction(q: np.ndarray) -> float:
    return float(np.mean(q == 0))
