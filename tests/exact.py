"""Exact-arithmetic helpers for the oracle pins (independent of the oracle).

Python Fractions give exact rational values; `f32_round` rounds one of them
to the nearest float32, ties to even, in one step.
"""
from fractions import Fraction

import numpy as np


def f32_round(fr):
    fr = Fraction(fr)
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    lsb = max(e - 23, -149)
    q = a / Fraction(2) ** lsb
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n) * 2.0 ** lsb)


def fmaf(a, b, c):
    """Single-rounding fused multiply-add on float32 values."""
    return f32_round(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))
