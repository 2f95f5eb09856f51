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
  {0, 1, 2}.  A 32-bit word holds 16 consecutive elements of a row, the even ones
  in the low half and the odd ones in the high half: element t of the word sits at
  bit 2*(t // 2) when t is even and at bit 16 + 2*(t // 2) when t is odd.  Words
  are ordered tile-interleaved: rows are taken in tiles of 16 (the last tile of a
  matrix holds the R <= 16 rows left); a tile stores its blocks in pairs (2h,
  2h+1), each pair as R * 4 units of 16 bytes, unit (row m of the tile, quarter
  kq) at index kq * R + m holding columns 32kq .. +32 of block 2h (2 words) then
  of block 2h+1 (2 words).  With an odd block count the last block is stored
  alone as R * 4 units of 8 bytes in the same order.  A stack of matrices is
  tiled matrix by matrix.
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
    """q int8 [M][K] in {-1,0,1} -> uint32 [M*K/16] in tile-interleaved order."""
    M, K = q.shape
    c = (q.astype(np.int64) + 1).reshape(M, K // 16, 16)
    words = (c << SHIFTS).sum(axis=-1).astype(np.uint32)    # [M][K/16], word w = columns 16w .. 16w+15
    G = K // BLOCK
    P = G // 2
    out = []
    for r0, R in _tiles(M, n_mats):
        blk = words[r0:r0 + R].reshape(R, G, 4, 2)                      # [row][block][quarter][word]
        pairs = blk[:, :2 * P].reshape(R, P, 2, 4, 2)                   # [row][pair][half][quarter][word]
        out.append(pairs.transpose(1, 3, 0, 2, 4).reshape(-1))          # [pair][quarter][row][half][word]
        if G % 2:
            out.append(blk[:, 2 * P].transpose(1, 0, 2).reshape(-1))    # [quarter][row][word]
    return np.concatenate(out)


def unpack_codes(words: np.ndarray, K: int, n_mats: int = 1) -> np.ndarray:
    """Tile-interleaved uint32 words (any shape, M*K/16 of them) -> q int8 [M][K];
    raises on the unused code 3."""
    flat = np.asarray(words, dtype=np.uint32).reshape(-1)
    M = flat.size * 16 // K
    G = K // BLOCK
    P = G // 2
    rows = np.empty((M, G, 4, 2), np.uint32)
    pos = 0
    for r0, R in _tiles(M, n_mats):
        n = P * R * 16
        rows[r0:r0 + R, :2 * P] = flat[pos:pos + n].reshape(P, 4, R, 2, 2).transpose(2, 0, 3, 1, 4).reshape(R, 2 * P, 4, 2)
        pos += n
        if G % 2:
            rows[r0:r0 + R, 2 * P] = flat[pos:pos + 8 * R].reshape(4, R, 2).transpose(1, 0, 2)
            pos += 8 * R
    shifts = SHIFTS.astype(np.uint32)
    c = (rows.reshape(M, K // 16)[..., None] >> shifts) & 3
    if np.any(c == 3):
        raise ValueError("invalid ternary code 3")
    return (c.astype(np.int8) - 1).reshape(M, K)


def dequant(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """fp64 [M][K] = q * s (exact)."""
    M, K = q.shape
    s = fp16_value(s_bits)
    return (q.reshape(M, K // BLOCK, BLOCK).astype(np.float64) * s[..., None]).reshape(M, K)


def pack(w_bits: np.ndarray, n_mats: int = 1) -> dict:
    """Packed sections {'codes', 'scales'} of a bf16 weight (n_mats stacked matrices)."""
    q, s = quantize(w_bits)
    return {"codes": pack_codes(q, n_mats), "scales": s}


def unpack_dequant(codes: np.ndarray, scales: np.ndarray, K: int, n_mats: int = 1) -> np.ndarray:
    """Dense fp64 weight from the packed sections."""
    M = np.asarray(codes).size * 16 // K
    return dequant(unpack_codes(codes, K, n_mats), np.asarray(scales).reshape(M, K // BLOCK))


def zero_fraction(q: np.ndarray) -> float:
    return float(np.mean(q == 0))
