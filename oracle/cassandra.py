"""Cassandra bit-split bf16 format: speculation data, verification data (oracle).

[Cassandra] §3.2 describes an offline transform in three steps, under the
invariant that speculation data + verification data reproduce every bit of the
original weights:

1. Value pruning with the Wanda score |w| * (L2 norm of the matching input
   channel's activations): the highest-scoring values are kept whole in the
   speculation data, the rest go to the verification data, and a bitmap marks
   which values were kept.
2. Mantissa truncation: a kept value keeps only the high bits of its 7-bit
   mantissa in the speculation data; the low bits go unchanged into the
   verification data, so restoring them is a concatenation.
3. Exponent compression ([Cassandra] §3.3, Cassandra-1): exponent values are
   ranked by frequency and rank r is written as r zero bits followed by a one,
   so every codeword ends in 1 and boundaries are found by counting zeros.
   The decoder works on fixed chunks of the stream with carried boundary state
   and a small rank -> exponent codebook ([Cassandra] §3.5).

The draft path ([Cassandra] §3.2, inference path b) reads speculation data only
and zero-fills both the pruned positions and the truncated mantissa bits; the
target path (path c) merges both parts back to the original bits.

Readings where the pages are silent (each listed in the design notes):
* Keep count per row is floor(K * 3 / 10); ties in score go to the lower k;
  activation norms are float32 and the score is formed exactly in fp64.
* 3 high mantissa bits are kept.  A kept value's speculation nibble is
  (S << 3) | (M >> 4); its verification nibble is M & 15.  Pruned values are
  stored raw (all 16 bits) in the verification data.
* Only kept values' exponents are unary coded (they are the speculation data).
  One codebook per matrix; equal counts rank the smaller exponent first; absent
  exponents get no rank.
* Bit order (parity unpinned by the pages, fixed here): the bitmap bit of flat
  element f = m*K + k is bit f % 32 of word f // 32; nibbles are packed eight to
  a 32-bit word, nibble i at bits 4*(i % 8) of word i // 8; the unary stream is
  LSB-first (stream bit p is bit p % 32 of word p // 32), codes in kept flat order.
* Tiles are consecutive 4096-element chunks of the flattened row-major weight
  (a tile may straddle rows; the last may be partial).  For tile t the table
  holds bitoff[t] (uint64, unary bits of all kept values before the tile) and
  kprefix[t] (uint32, kept values before the tile), with a final sentinel.
* A pruned position decodes to +0.0 (bits 0x0000) on the draft path.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_fields

TILE = 4096
MANT_HI_BITS = 3


def keep_count(K: int, num: int = 3, den: int = 10) -> int:
    return (K * num) // den


def keep_mask(w_bits: np.ndarray, norms: np.ndarray, num: int = 3, den: int = 10,
              row_chunk: int = 256) -> np.ndarray:
    """bool [M][K]: per row, the floor(K*num/den) highest Wanda scores |w| * norm[k]."""
    M, K = w_bits.shape
    if norms.shape != (K,):
        raise ValueError("norms must have shape [K]")
    nk = keep_count(K, num, den)
    out = np.zeros((M, K), dtype=bool)
    nrm = norms.astype(np.float32).astype(np.float64)
    for r0 in range(0, M, row_chunk):
        r1 = min(M, r0 + row_chunk)
        b = w_bits[r0:r1].astype(np.int64)
        ex = (b >> 7) & 0xFF
        if np.any(ex == 255):
            raise ValueError("bf16 Inf/NaN in input")
        mag = np.where(ex > 0, np.ldexp((128 + (b & 0x7F)).astype(np.float64), ex - 134),
                       np.ldexp((b & 0x7F).astype(np.float64), -133))
        score = mag * nrm[None, :]
        order = np.argsort(-score, axis=1, kind="stable")[:, :nk]
        rows = np.repeat(np.arange(r1 - r0), nk)
        out[r0 + rows, order.reshape(-1)] = True
    return out


def pack_bits_lsb(flags: np.ndarray) -> np.ndarray:
    """bool [n] -> uint32 words, flag i at bit i % 32 of word i // 32 (zero padded)."""
    flags = np.asarray(flags, dtype=np.uint8).reshape(-1)
    n = flags.size
    pad = (-n) % 32
    if pad:
        flags = np.concatenate([flags, np.zeros(pad, np.uint8)])
    return np.packbits(flags, bitorder="little").view(np.uint32).copy()


def unpack_bits_lsb(words: np.ndarray, n: int) -> np.ndarray:
    return np.unpackbits(np.ascontiguousarray(words, dtype=np.uint32).view(np.uint8),
                         bitorder="little")[:n].astype(bool)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """uint8 [n] in [0, 15] -> uint32 words, nibble i at bits 4*(i % 8) of word i // 8."""
    nib = np.asarray(nib, dtype=np.int64).reshape(-1)
    pad = (-nib.size) % 8
    if pad:
        nib = np.concatenate([nib, np.zeros(pad, np.int64)])
    shifts = 4 * np.arange(8, dtype=np.int64)
    return (nib.reshape(-1, 8) << shifts).sum(axis=1).astype(np.uint32)


def unpack_nibbles(words: np.ndarray, n: int) -> np.ndarray:
    shifts = 4 * np.arange(8, dtype=np.uint32)
    return ((np.asarray(words, np.uint32)[:, None] >> shifts) & 15).reshape(-1)[:n].astype(np.uint8)


def build_codebook(kept_exps: np.ndarray) -> np.ndarray:
    """uint8 [n_sym]: exponents present among kept values, by (-count, exponent)."""
    counts = np.bincount(np.asarray(kept_exps, np.int64), minlength=256)
    present = np.flatnonzero(counts)
    order = sorted(present.tolist(), key=lambda e: (-int(counts[e]), e))
    return np.array(order, dtype=np.uint8)


def unary_encode(ranks: np.ndarray):
    """(stream uint32 words, code lengths int64): rank r -> r zeros then a one, LSB-first."""
    ranks = np.asarray(ranks, dtype=np.int64)
    lengths = ranks + 1
    ends = np.cumsum(lengths) - 1
    total = int(lengths.sum())
    bits = np.zeros(total, dtype=bool)
    bits[ends] = True
    return pack_bits_lsb(bits), lengths


def unary_decode(stream: np.ndarray, n_codes: int, bit0: int = 0) -> np.ndarray:
    """Ranks of the first ``n_codes`` codewords starting at stream bit ``bit0``."""
    bits = unpack_bits_lsb(stream, stream.size * 32)[bit0:]
    ones = np.flatnonzero(bits)[:n_codes]
    if ones.size < n_codes:
        raise ValueError("unary stream ends before the last codeword")
    return np.diff(ones, prepend=-1) - 1


def tile_table(keep_flat: np.ndarray, lengths: np.ndarray, tile: int = TILE):
    """(bitoff uint64 [T+1], kprefix uint32 [T+1]) over flat tiles of ``tile`` elements."""
    n = keep_flat.size
    T = -(-n // tile)
    kept_before = np.concatenate([[0], np.cumsum(keep_flat, dtype=np.int64)])   # [n+1]
    bits_before = np.concatenate([[0], np.cumsum(lengths, dtype=np.int64)])      # [kept+1]
    starts = np.minimum(np.arange(T + 1, dtype=np.int64) * tile, n)
    kp = kept_before[starts]
    return bits_before[kp].astype(np.uint64), kp.astype(np.uint32)


def pack(w_bits: np.ndarray, norms: np.ndarray, num: int = 3, den: int = 10) -> dict:
    """All sections of the Cassandra format for a bf16 weight [M][K]."""
    M, K = w_bits.shape
    keep = keep_mask(w_bits, norms, num, den)
    flat = w_bits.reshape(-1)
    kf = keep.reshape(-1)
    S, E, Mn = bf16_fields(flat)
    kS, kE, kM = S[kf], E[kf], Mn[kf]
    spec_nib = (kS << 3) | (kM >> (7 - MANT_HI_BITS))
    lo_nib = kM & ((1 << (7 - MANT_HI_BITS)) - 1)
    cb = build_codebook(kE)
    rank_of = np.full(256, -1, dtype=np.int64)
    rank_of[cb.astype(np.int64)] = np.arange(cb.size)
    ranks = rank_of[kE]
    stream, lengths = unary_encode(ranks)
    bitoff, kprefix = tile_table(kf, lengths)
    return {
        "bitmap": pack_bits_lsb(kf),
        "spec_nib": pack_nibbles(spec_nib),
        "unary": stream,
        "codebook": cb,
        "bitoff": bitoff,
        "kprefix": kprefix,
        "lo_nib": pack_nibbles(lo_nib),
        "pruned": flat[~kf].astype(np.uint16),
        "n_kept": int(kf.sum()),
        "n_sym": int(cb.size),
        "unary_bits": int(lengths.sum()),
    }


def _kept_positions(sec: dict, n: int) -> np.ndarray:
    return np.flatnonzero(unpack_bits_lsb(sec["bitmap"], n))


def spec_decode(sec: dict, M: int, K: int) -> np.ndarray:
    """Draft weights from speculation data only: bf16 bits [M][K].

    Kept: (S << 15) | (E << 7) | (M_hi << 4); pruned: +0.0."""
    n = M * K
    pos = _kept_positions(sec, n)
    nk = pos.size
    ranks = unary_decode(sec["unary"], nk)
    cb = np.asarray(sec["codebook"], dtype=np.int64)
    if ranks.size and ranks.max() >= cb.size:
        raise ValueError("unary rank outside the codebook")
    E = cb[ranks]
    nib = unpack_nibbles(sec["spec_nib"], nk).astype(np.int64)
    bits = ((nib >> 3) << 15) | (E << 7) | ((nib & 7) << (7 - MANT_HI_BITS))
    out = np.zeros(n, dtype=np.uint16)
    out[pos] = bits.astype(np.uint16)
    return out.reshape(M, K)


def restore(sec: dict, M: int, K: int) -> np.ndarray:
    """Target weights from speculation + verification data: bf16 bits [M][K]."""
    n = M * K
    keep = unpack_bits_lsb(sec["bitmap"], n)
    spec = spec_decode(sec, M, K).reshape(-1)
    nk = int(keep.sum())
    lo = unpack_nibbles(sec["lo_nib"], nk).astype(np.uint16)
    out = np.empty(n, dtype=np.uint16)
    out[keep] = spec[keep] | lo
    out[~keep] = np.asarray(sec["pruned"], dtype=np.uint16)[: n - nk]
    return out.reshape(M, K)


def stats(sec: dict, M: int, K: int) -> dict:
    """Exponent entropy and average unary length over kept values, bits per weight."""
    n = M * K
    nk = sec["n_kept"]
    ranks = unary_decode(sec["unary"], nk)
    p = np.bincount(ranks) / nk
    p = p[p > 0]
    spec_bits = n + 4 * nk + sec["unary_bits"]
    return {
        "entropy_bits": float(-(p * np.log2(p)).sum()),
        "unary_avg_bits": float(sec["unary_bits"] / nk),
        "kept": nk,
        "spec_bpw": spec_bits / n,
        "verify_bpw": (4 * nk + 16 * (n - nk)) / n,
    }
