"""Block-ternary weights with all-zero blocks left out of storage (oracle).

Test infrastructure only: the library never imports this module.

[Bonsai2] §3.4 and §5.5: a 128-value block with no surviving weight gets scale
1, is flagged all-zero in the package, and its 128 zero codes are not stored.
[Bonsai2] §1.3 / §3.3: the sparsity is structured by block, which is what lets
storage and reads skip it.  The quantizer is the one of ``oracle.ternary``
(§1.2); this module adds only the flag and the compacted code stream.

Readings where the pages are silent (each listed in the design notes):
* A block is "all-zero" when all its 128 codes are q = 0.  Under absmean a block
  with any non-zero weight has max|w| >= scale, so some code is +-1: the flag
  is set exactly for blocks whose weights are all zero.
* The pages give no byte format for the flag or for the skipped stream (parity
  unpinned by the pages beyond the invariants tested), fixed here:
  - "scales" fp16 [M][K/128] as in the dense format (1.0 for a flagged block);
  - "slabs" uint32 [tiles][K/128]: one word per (16-row tile, block column g);
    bit m (m < R) is set when tile row m's block is stored (not all-zero), so the
    pages' all-zero flag is the clear bit; bits 16..31 hold the blocks stored in
    this tile before block column g;
  - "tile_base" uint32 [tiles + 1]: blocks stored before each tile (the last
    entry is the total);
  - "codes" uint32: the stored blocks, 32 bytes each, tile by tile and block
    column by block column; within one (tile, g) the nz stored blocks, ranked r
    = 0.. by tile row, are laid out as 4 * nz units of 8 bytes, unit (r, kq) at
    index kq * nz + r holding columns 32kq .. +32 of the block (2 words, the
    dense format's word encoding).  With no block flagged this is the dense
    format's layout of a lone block (units of 8 bytes, unit (m, kq) at kq R + m).
"""
from __future__ import annotations

import numpy as np

from . import ternary

BLOCK = ternary.BLOCK
TILE = ternary.TILE


def zero_blocks(q: np.ndarray) -> np.ndarray:
    """bool [M][K/128]: the block's codes are all q = 0 ([Bonsai2] §3.4)."""
    M, K = q.shape
    return np.all(q.reshape(M, K // BLOCK, BLOCK) == 0, axis=-1)


def _block_words(q: np.ndarray) -> np.ndarray:
    """uint32 [M][K/128][4][2]: the 8 words of each block, quarter by quarter,
    in the dense format's word encoding (16 elements a word)."""
    M, K = q.shape
    c = (q.astype(np.int64) + 1).reshape(M, K // 16, 16)
    words = (c << ternary.SHIFTS).sum(axis=-1).astype(np.uint32)
    return words.reshape(M, K // BLOCK, 4, 2)


def pack_sections(q: np.ndarray, s_bits: np.ndarray) -> dict:
    """Sections {'codes', 'scales', 'slabs', 'tile_base'} from codes and scales."""
    M, K = q.shape
    G = K // BLOCK
    if 16 * G > 1 << 16:
        raise ValueError("K too large for the 16-bit in-tile block offset")
    words = _block_words(q)
    stored = ~zero_blocks(q)
    tiles = (M + TILE - 1) // TILE
    slabs = np.zeros((tiles, G), np.uint32)
    tile_base = np.zeros(tiles + 1, np.uint32)
    out = []
    total = 0
    for t in range(tiles):
        r0 = t * TILE
        R = min(TILE, M - r0)
        tile_base[t] = total
        in_tile = 0
        for g in range(G):
            rows = [m for m in range(R) if stored[r0 + m, g]]
            mask = sum(1 << m for m in rows)
            slabs[t, g] = mask | (in_tile << 16)
            for kq in range(4):
                for m in rows:
                    out.append(words[r0 + m, g, kq])
            in_tile += len(rows)
        total += in_tile
    tile_base[tiles] = total
    codes = np.concatenate(out).astype(np.uint32) if out else np.zeros(0, np.uint32)
    return {"codes": codes, "scales": np.asarray(s_bits, np.uint16), "slabs": slabs, "tile_base": tile_base}


def pack(w_bits: np.ndarray) -> dict:
    """Packed sections of a bf16 weight [M][K]: the [Bonsai2] §1.2 quantizer, then
    the all-zero blocks dropped."""
    q, s = ternary.quantize(w_bits)
    return pack_sections(q, s)


def unpack_codes(sec: dict, M: int, K: int) -> np.ndarray:
    """q int8 [M][K] from the sections: flagged blocks read as zeros; raises on an
    inconsistent table or the unused code 3."""
    G = K // BLOCK
    codes = np.asarray(sec["codes"], np.uint32).reshape(-1)
    slabs = np.asarray(sec["slabs"], np.uint32).reshape(-1, G)
    base = np.asarray(sec["tile_base"], np.uint32).reshape(-1)
    tiles = (M + TILE - 1) // TILE
    if slabs.shape[0] != tiles or base.size != tiles + 1:
        raise ValueError("table sizes do not match the shape")
    blocks = np.full((M, G, 4, 2), 0x55555555, np.uint32)    # code 1 (q = 0) everywhere
    for t in range(tiles):
        r0 = t * TILE
        R = min(TILE, M - r0)
        in_tile = 0
        for g in range(G):
            mask = int(slabs[t, g]) & 0xFFFF
            if mask >> R or (int(slabs[t, g]) >> 16) != in_tile:
                raise ValueError("bad slab word")
            rows = [m for m in range(R) if mask >> m & 1]
            nz = len(rows)
            start = (int(base[t]) + in_tile) * 8               # words
            for r, m in enumerate(rows):
                for kq in range(4):
                    u = start + 2 * (kq * nz + r)
                    blocks[r0 + m, g, kq] = codes[u:u + 2]
            in_tile += nz
        if int(base[t + 1]) != int(base[t]) + in_tile:
            raise ValueError("bad tile base")
    if codes.size != 8 * int(base[tiles]):
        raise ValueError("codes size does not match the stored blocks")
    c = (blocks.reshape(M, K // 16)[..., None] >> ternary.SHIFTS.astype(np.uint32)) & 3
    if np.any(c == 3):
        raise ValueError("invalid ternary code 3")
    return (c.astype(np.int8) - 1).reshape(M, K)


def unpack_dequant(sec: dict, M: int, K: int) -> np.ndarray:
    """Dense fp64 weight from the sections."""
    return ternary.dequant(unpack_codes(sec, M, K), np.asarray(sec["scales"]).reshape(M, K // BLOCK))


def stored_bytes(sec: dict) -> int:
    """Bytes of all four sections (what a GEMV over them reads)."""
    return sum(int(np.asarray(sec[k]).nbytes) for k in ("codes", "scales", "slabs", "tile_base"))
