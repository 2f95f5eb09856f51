"""MX-32 shared-exponent variant of the verify-side weights (oracle).

[Cassandra] §3.3 (Cassandra-2): a group of adjacent values (32) shares the
largest exponent in the group, and each value's mantissa is shifted right by
the difference between that shared exponent and its own; small values lose low
bits, so the format is slightly lossy but decodes faster.

Readings (the page gives no bit layout; parity unpinned beyond the invariants
tested: elements at the shared exponent are exact, |mx| <= |w|, the error is
below one unit of the shared exponent's last place, an all-zero group has
magnitude 0):
* Groups are 32 consecutive k of one row of the restored bf16 weight.
* Effective exponent e' = max(E, 1) (a subnormal behaves as exponent 1);
  X = max e' over the group; the significand is 128 | M for E >= 1 and M for
  E = 0; the stored magnitude is significand >> (X - e') (0 when the shift is 8
  or more), i.e. the right shift truncates.
* Sections: shared exponent uint8 [M][K/32], sign word uint32 [M][K/32] with
  bit i the sign of element i of the group, magnitude uint8 [M][K].
* Value = (-1)^S * mag * 2^(X - 134); it is exactly representable in bf16.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_fields

GROUP = 32


def encode(w_bits: np.ndarray) -> dict:
    M, K = w_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    S, E, Mn = bf16_fields(w_bits)
    if np.any(E == 255):
        raise ValueError("bf16 Inf/NaN in input")
    ep = np.maximum(E, 1).reshape(M, K // GROUP, GROUP)
    X = ep.max(axis=-1)
    sig = np.where(E >= 1, 128 | Mn, Mn).reshape(M, K // GROUP, GROUP)
    d = X[..., None] - ep
    mag = np.where(d >= 8, 0, sig >> np.minimum(d, 7))
    signs = (S.reshape(M, K // GROUP, GROUP) << np.arange(GROUP)).sum(axis=-1)
    return {
        "mx_exp": X.astype(np.uint8),
        "mx_sign": signs.astype(np.uint32),
        "mx_mag": mag.reshape(M, K).astype(np.uint8),
    }


def value(sec: dict, M: int, K: int) -> np.ndarray:
    """fp64 [M][K] values of the MX-32 sections."""
    X = sec["mx_exp"].astype(np.int64).reshape(M, K // GROUP, 1)
    sgn = (sec["mx_sign"].astype(np.int64).reshape(M, K // GROUP, 1) >> np.arange(GROUP)) & 1
    mag = sec["mx_mag"].astype(np.float64).reshape(M, K // GROUP, GROUP)
    v = np.ldexp(mag, X - 134)
    return np.where(sgn == 1, -v, v).reshape(M, K)
