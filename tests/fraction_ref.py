"""Exact rational arithmetic and IEEE round-to-nearest-even, written from the IEEE 754 rules.

Used only by tests to pin the oracle's float64/numpy arithmetic against exact
values. Independent of ``oracle/`` (imports nothing from it).
"""
from __future__ import annotations

import math
from fractions import Fraction

# (significand bits incl. the implicit one, minimum normal exponent, maximum exponent)
FORMATS = {
    "f32": (24, -126, 127),
    "bf16": (8, -126, 127),
    "f64": (53, -1022, 1023),
}


def exact(v: float) -> Fraction:
    return Fraction(float(v))


def round_fraction(q: Fraction, fmt: str) -> float:
    """Round an exact rational to the nearest value of ``fmt`` (ties to even), as a Python float.

    Exact zero returns +0.0 (signs of zero are handled by callers). Values at or
    past the overflow threshold return +-inf.
    """
    p, emin, emax = FORMATS[fmt]
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    # e = floor(log2(a)), exactly
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    m = math.floor(n)
    rem = n - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    r = m * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(r)


def dot_exact(p, q) -> Fraction:
    return sum((exact(a) * exact(b) for a, b in zip(p, q)), Fraction(0))
