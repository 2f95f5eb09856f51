"""bf16 and fp16 bit fields, values and rounding (oracle; test infrastructure only).

[Cassandra] §3.1: a bf16 number is a sign bit S, an 8-bit biased exponent E and
a 7-bit mantissa M; a normal value is (-1)^S * 2^(E-127) * 1.M.  The oracle uses
the IEEE reading for the cases the page does not print: E = 0 is a subnormal
(-1)^S * M * 2^-133 and E = 255 (Inf / NaN) is rejected.

fp16 rounding is written from the IEEE 754 binary16 definition (round to nearest,
ties to even, subnormals kept, overflow to infinity) acting on an exact float64
value, so no intermediate float32 rounding is involved.
"""
from __future__ import annotations

import numpy as np


def bf16_fields(b):
    """(S, E, M) integer arrays of bf16 bit patterns ``b``."""
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    return b >> 15, (b >> 7) & 0xFF, b & 0x7F


def bf16_value(b) -> np.ndarray:
    """Exact float64 value of bf16 bits.  Raises ValueError on E == 255."""
    S, E, M = bf16_fields(b)
    if np.any(E == 255):
        raise ValueError("bf16 Inf/NaN in input")
    sig = np.where(E > 0, 128 + M, M).astype(np.float64)
    ex = np.where(E > 0, E - 134, -133)
    v = np.ldexp(sig, ex)
    return np.where(S == 1, -v, v)


def fp16_rne(v) -> np.ndarray:
    """IEEE binary16 bits of float64 ``v`` rounded to nearest, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN")
    sign = np.signbit(v).astype(np.uint16) << 15
    a = np.abs(v)
    out = np.zeros(a.shape, dtype=np.uint16)
    nz = a > 0
    # unbiased exponent e with 2^e <= a < 2^(e+1)
    _, fx = np.frexp(np.where(nz, a, 1.0))
    e = fx.astype(np.int64) - 1
    sub = nz & (e < -14)
    nrm = nz & ~sub
    # subnormal range: quantum 2^-24, the integer is the whole 10-bit field
    if np.any(sub):
        m = np.rint(np.ldexp(a[sub], 24)).astype(np.int64)
        out[sub] = m.astype(np.uint16)          # m == 1024 is exactly the smallest normal
    if np.any(nrm):
        en = e[nrm]
        m = np.rint(np.ldexp(a[nrm], 10 - en)).astype(np.int64)   # in [1024, 2048]
        carry = m == 2048
        en = np.where(carry, en + 1, en)
        m = np.where(carry, 1024, m)
        biased = en + 15
        bits = (biased << 10) | (m - 1024)
        bits = np.where(biased >= 31, 0x7C00, bits)
        out[nrm] = bits.astype(np.uint16)
    return out | sign


def fp16_value(h) -> np.ndarray:
    """Exact float64 value of fp16 bits (finite only)."""
    h = np.asarray(h, dtype=np.uint16).astype(np.int64)
    S, E, M = h >> 15, (h >> 10) & 0x1F, h & 0x3FF
    if np.any(E == 31):
        raise ValueError("fp16 Inf/NaN")
    v = np.where(E > 0, np.ldexp((1024 + M).astype(np.float64), E - 25),
                 np.ldexp(M.astype(np.float64), -24))
    return np.where(S == 1, -v, v)


FP16_ONE = np.uint16(0x3C00)
