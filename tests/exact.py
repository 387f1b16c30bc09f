"""Exact rational arithmetic used by the oracle pins.

Independent of oracle/: values are Python Fractions, and rounding to a binary
format is done from the definition (pick the nearest representable value,
ties to an even significand) with integer arithmetic, so a slip in the
oracle's float32/float64 handling cannot hide behind the same slip here.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# (precision p incl. hidden bit, minimum normal exponent, maximum exponent)
FORMATS = {
    "f32": (24, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def _floor_log2(q: Fraction) -> int:
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_rational(q: Fraction, fmt: str) -> Fraction:
    """q rounded to the binary format, round half to even (overflow -> inf not
    handled: callers stay in range)."""
    if q == 0:
        return Fraction(0)
    p, emin, emax = FORMATS[fmt]
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    m = a / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    assert r < Fraction(2) ** (emax + 1), "overflow"
    return sign * r


def next_up(c: Fraction, fmt: str) -> Fraction:
    p, emin, _ = FORMATS[fmt]
    return c + Fraction(2) ** (max(_floor_log2(c), emin) - p + 1)


def next_down(c: Fraction, fmt: str) -> Fraction:
    """Largest representable value below c > 0 (c representable)."""
    p, emin, _ = FORMATS[fmt]
    e = _floor_log2(c)
    if c == Fraction(2) ** e:  # a power of two: the gap below is half as wide
        e -= 1
    return c - Fraction(2) ** (max(e, emin) - p + 1)


def round_sqrt(q: Fraction, fmt: str) -> Fraction:
    """sqrt(q) rounded to nearest in the format (q > 0). Start from a float
    guess and move while sqrt(q) lies beyond a midpoint, comparing squares of
    midpoints with q exactly. (sqrt(q) of a representable q never equals a
    midpoint exactly: a midpoint's square has more significant bits than q.)"""
    c = round_rational(Fraction(float(np.sqrt(float(q)))), fmt)
    while True:
        up = next_up(c, fmt)
        if q > ((c + up) / 2) ** 2:
            c = up
            continue
        dn = next_down(c, fmt)
        if dn > 0 and q < ((c + dn) / 2) ** 2:
            c = dn
            continue
        return c


def f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def to_f32(q: Fraction) -> np.float32:
    return np.float32(float(round_rational(q, "f32")))
