"""Exact-arithmetic helpers for pinning the oracle (test code only).

Values are carried as fractions.Fraction and rounded to binary32 once, with
round-to-nearest-even, including the subnormal range and overflow. This is
the mathematical definition of "compute exactly, round once", written
independently of the oracle's C code.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np


def frac(x) -> Fraction:
    """Exact value of a float / numpy float (any finite binary value)."""
    return Fraction(float(x))


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_f32(q: Fraction, negative_zero: bool = False) -> float:
    """Correctly rounded (RNE) binary32 value of the exact rational q."""
    if q == 0:
        return -0.0 if negative_zero else 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = _floor_log2(a)
    qexp = max(e, -126) - 23
    scaled = a / (Fraction(2) ** qexp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** qexp
    if val >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(val)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", np.float32(x)))[0]


def same_f32(a, b) -> bool:
    """Bit equality of two binary32 values (distinguishes -0 from +0; NaN == NaN)."""
    a32, b32 = np.float32(a), np.float32(b)
    if np.isnan(a32) and np.isnan(b32):
        return True
    return f32_bits(a32) == f32_bits(b32)


def same_val(a, b) -> bool:
    """Bit equality of two binary32 values, except that +0 and -0 compare
    equal (used where the sign of an exact zero result is fixed by IEEE
    arithmetic on the stated operations rather than by the format)."""
    if float(a) == 0.0 and float(b) == 0.0:
        return True
    return same_f32(a, b)
