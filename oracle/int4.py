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
  (0 is never written).  A 32-bit word holds 8 consecutive elements of a row,
  the even ones in the low half and the odd ones in the high half: element t of
  the word sits at bit 4*(t // 2) when t is even and at bit 16 + 4*(t // 2) when
  t is odd.  Words are ordered tile-interleaved: rows are taken in tiles of 16
  (the last tile of a matrix holds the R <= 16 rows left); a tile stores its
  groups in order, and group g of a tile is R * 4 units of 16 bytes, unit
  (row m of the tile, quarter kq) at index kq * R + m holding columns
  128g + 32kq .. +32 as 4 words.  A stack of matrices is tiled matrix by matrix.
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


TILE = 16


def _tiles(M: int, n_mats: int):
    """(first row, rows) of each 16-row tile, matrix by matrix."""
    if M % n_mats:
        raise ValueError("rows not divisible by n_mats")
    Mm = M // n_mats
    for mat in range(n_mats):
        for t0 in range(0, Mm, TILE):
            yield mat * Mm + t0, min(TILE, Mm - t0)


def pack_codes(q: np.ndarray, n_mats: int = 1) -> np.ndarray:
    """q int8 [M][K] in [-7, 7] -> uint32 [M*K/8] in tile-interleaved order."""
    M, K = q.shape
    c = (q.astype(np.int64) + 8).reshape(M, K // 8, 8)
    words = (c << SHIFTS).sum(axis=-1).astype(np.uint32)    # [M][K/8], word w = columns 8w .. 8w+7
    G = K // GROUP
    out = []
    for r0, R in _tiles(M, n_mats):
        blk = words[r0:r0 + R].reshape(R, G, 4, 4)           # [row][group][quarter][word]
        out.append(blk.transpose(1, 2, 0, 3).reshape(-1))    # [group][quarter][row][word]
    return np.concatenate(out)


def unpack_codes(words: np.ndarray, K: int, n_mats: int = 1) -> np.ndarray:
    """Tile-interleaved uint32 words (any shape, M*K/8 of them) -> q int8 [M][K];
    raises on the unused code 0."""
    flat = np.asarray(words, dtype=np.uint32).reshape(-1)
    M = flat.size * 8 // K
    G = K // GROUP
    rows = np.empty((M, K // 8), np.uint32)
    pos = 0
    for r0, R in _tiles(M, n_mats):
        n = R * K // 8
        rows[r0:r0 + R] = flat[pos:pos + n].reshape(G, 4, R, 4).transpose(2, 0, 1, 3).reshape(R, K // 8)
        pos += n
    shifts = SHIFTS.astype(np.uint32)
    c = (rows[..., None] >> shifts) & 15
    if np.any(c == 0):
        raise ValueError("invalid int4 code 0")
    return (c.astype(np.int8) - 8).reshape(M, K)


def dequant(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    M, K = q.shape
    s = fp16_value(s_bits)
    return (q.reshape(M, K // GROUP, GROUP).astype(np.float64) * s[..., None]).reshape(M, K)


def pack(w_bits: np.ndarray, n_mats: int = 1) -> dict:
    q, s = quantize(w_bits)
    return {"codes": pack_codes(q, n_mats), "scales": s}


def unpack_dequant(codes: np.ndarray, scales: np.ndarray, K: int, n_mats: int = 1) -> np.ndarray:
    M = np.asarray(codes).size * 8 // K
    return dequant(unpack_codes(codes, K, n_mats), np.asarray(scales).reshape(M, K // GROUP))
