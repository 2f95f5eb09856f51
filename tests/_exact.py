"""Exact rational helpers for brute-force pins of the oracle.

Independent of ``oracle.bits``: bf16 values come from numpy's float32 view of the
bits shifted into the high half, and fp16 rounding is done on
``fractions.Fraction`` with integer arithmetic only.
"""
from fractions import Fraction

import numpy as np


def bf16_frac(b: int) -> Fraction:
    f = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def _round_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def round_half_even(v: Fraction) -> int:
    return -_round_half_even(-v) if v < 0 else _round_half_even(v)


def fp16_frac(v: Fraction) -> Fraction:
    """Nearest binary16 value to v (ties to even), as a Fraction; inf -> None."""
    if v == 0:
        return Fraction(0)
    neg = v < 0
    a = -v if neg else v
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    quantum = Fraction(2) ** (max(e, -14) - 10)
    n = _round_half_even(a / quantum)
    r = n * quantum
    if r >= 65536 or r > 65504:
        return None
    return -r if neg else r


def fp16_bits_value(h: int) -> Fraction:
    f = np.array([h], dtype=np.uint16).view(np.float16)[0]
    return Fraction(float(f))
