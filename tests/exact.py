"""Exact rational arithmetic helpers for the oracle pins (no oracle code)."""
from fractions import Fraction
import math

import numpy as np


def rn32(q):
    """Round a rational to the nearest binary32, ties to even."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)                 # below 2^-126 the spacing stays 2^-149
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    n = math.floor(m)
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))


def round_half_even(q):
    q = Fraction(q)
    n = math.floor(q)
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def F(x):
    """Exact rational value of a finite float."""
    return Fraction(float(x))


def bits32(x):
    return int(np.float32(x).view(np.uint32))


def from_bits32(u):
    return np.array([u], np.uint32).view(np.float32)[0]
