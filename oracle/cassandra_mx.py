"""Cassandra-2 speculation data: the kept values' exponents as MX-32 (oracle).

Test infrastructure only: the library never imports this module.

[Cassandra] §3.3 names two ways to code the exponents of the speculation data:
Cassandra-1 ranks exponent values by frequency and writes each as a unary code
(lossless, decoded by counting zeros); Cassandra-2 uses the MX format instead:
a group of adjacent values (for example 32) shares its largest exponent, and
each value's mantissa is shifted right by the difference between the shared
exponent and its own.  That drops low bits of the smaller values (slightly
lossy) but needs no per-value code parsing, so it decodes faster.  Pruning
(Wanda, the bitmap) and the 3-bit mantissa truncation of §3.2 are unchanged, so
they come from ``oracle.cassandra``.

Readings where the page is silent (each listed in the design notes):
* The 32 adjacent values are 32 consecutive kept values of the speculation
  stream, in kept flat order (a group may cross rows and tiles); the last group
  may be short.
* A kept value has sign S, exponent E and the 3 kept mantissa bits H.  Its
  significand is 8 + H (the implicit one) when E >= 1 and H when E = 0, with
  effective exponent e' = max(E, 1), so that it equals sig * 2^(e' - 130).  The
  shared exponent X is the largest e' of the group; the stored magnitude is
  sig >> (X - e'), truncating (0 once the shift reaches 4).  The draft value is
  (-1)^S * mag * 2^(X - 130), exact in bf16; a pruned position is +0.0.
* Byte format (parity unpinned by the pages beyond the tested invariants):
  "bitmap" as Cassandra-1; "mx_nib" uint32, magnitude nibble of kept value i at
  bits 4*(i % 8) of word i // 8; "mx_sign" uint32, sign of kept value i at bit
  i % 32 of word i // 32 (one word per group); "mx_exp" uint8, X of each group;
  "kprefix" uint32 [T+1], kept values before each 4096-element flat tile.
* The format holds speculation data only: the page fixes no verification side
  for the lossy code, so a target keeps reading a restoring format.
"""
from __future__ import annotations

import numpy as np

from . import cassandra
from .bits import bf16_fields

GROUP = 32
SHIFT_BIAS = 130          # value = mag * 2^(X - 130)


def kept_fields(w_bits: np.ndarray, keep: np.ndarray):
    """(S, E, H) of the kept values in kept flat order: sign, exponent, 3 high
    mantissa bits."""
    S, E, Mn = bf16_fields(w_bits.reshape(-1)[keep.reshape(-1)])
    return S.astype(np.int64), E.astype(np.int64), (Mn >> (7 - cassandra.MANT_HI_BITS)).astype(np.int64)


def mx_encode(S: np.ndarray, E: np.ndarray, H: np.ndarray):
    """(mag, X per group, sign) of kept values given their fields."""
    n = S.size
    ep = np.maximum(E, 1)
    sig = np.where(E >= 1, 8 + H, H)
    ng = (n + GROUP - 1) // GROUP
    padded = np.zeros(ng * GROUP, np.int64)           # e' >= 1, so padding never wins
    padded[:n] = ep
    X = padded.reshape(ng, GROUP).max(axis=1)
    d = X[np.arange(n) // GROUP] - ep
    mag = np.where(d >= 4, 0, sig >> np.minimum(d, 4))
    return mag, X, S


def pack_spec(w_bits: np.ndarray, norms: np.ndarray, num: int = 3, den: int = 10) -> dict:
    """Speculation sections of the MX-32 exponent code for a bf16 weight [M][K]."""
    M, K = w_bits.shape
    keep = cassandra.keep_mask(w_bits, norms, num, den)
    S, E, H = kept_fields(w_bits, keep)
    if np.any(E == 255):
        raise ValueError("bf16 Inf/NaN kept")
    mag, X, sign = mx_encode(S, E, H)
    n = mag.size
    ng = X.size
    sbits = np.zeros(ng * GROUP, np.uint64)
    sbits[:n] = sign.astype(np.uint64) << (np.arange(n) % GROUP).astype(np.uint64)
    sign_words = sbits.reshape(ng, GROUP).sum(axis=1).astype(np.uint32)    # distinct bits: sum = or
    kf = keep.reshape(-1)
    T = (kf.size + cassandra.TILE - 1) // cassandra.TILE
    before = np.concatenate([[0], np.cumsum(kf, dtype=np.int64)])
    kprefix = before[np.minimum(np.arange(T + 1) * cassandra.TILE, kf.size)].astype(np.uint32)
    return {
        "bitmap": cassandra.pack_bits_lsb(kf),
        "mx_nib": cassandra.pack_nibbles(mag),
        "mx_sign": sign_words,
        "mx_exp": X.astype(np.uint8),
        "kprefix": kprefix,
        "n_kept": int(n),
    }


def draft_values(sec: dict, n_kept: int) -> np.ndarray:
    """fp64 draft values of the kept values, in kept order."""
    mag = cassandra.unpack_nibbles(sec["mx_nib"], n_kept).astype(np.int64)
    i = np.arange(n_kept)
    X = np.asarray(sec["mx_exp"], dtype=np.int64)[i // GROUP]
    S = (np.asarray(sec["mx_sign"], dtype=np.uint32)[i // GROUP] >> (i % GROUP).astype(np.uint32)) & 1
    v = np.ldexp(mag.astype(np.float64), X - SHIFT_BIAS)
    return np.where(S == 1, -v, v)


def spec_decode(sec: dict, M: int, K: int) -> np.ndarray:
    """Draft weights: bf16 bits [M][K]; a kept value with magnitude 0 keeps its
    sign (-0.0), a pruned position is +0.0."""
    n = M * K
    keep = cassandra.unpack_bits_lsb(sec["bitmap"], n)
    nk = int(keep.sum())
    v = draft_values(sec, nk)
    bits = (np.abs(v).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact: <= 4 significant bits
    i = np.arange(nk)
    S = (np.asarray(sec["mx_sign"], dtype=np.uint32)[i // GROUP] >> (i % GROUP).astype(np.uint32)) & 1
    bits = bits | (S.astype(np.uint16) << 15)
    out = np.zeros(n, dtype=np.uint16)
    out[keep] = bits
    return out.reshape(M, K)


def spec_bits(sec: dict) -> int:
    """Meaningful bits of the speculation sections."""
    return 8 * sum(int(np.asarray(sec[k]).nbytes) for k in ("bitmap", "mx_nib", "mx_sign", "mx_exp", "kprefix"))
