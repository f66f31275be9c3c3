"""Exact rational -> binary32 rounding for test expectations (no oracle code)."""

from fractions import Fraction

import numpy as np


def round_f32(q: Fraction) -> np.float32:
    """Nearest binary32 to the rational q, ties to even (normal range only)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # normalise so that 2^23 <= a / 2^(e-23) < 2^24
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "normal range only"
    scaled = a / Fraction(2) ** (e - 23)
    r = scaled.numerator // scaled.denominator
    rem = scaled - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    return np.float32(sign * float(Fraction(r) * Fraction(2) ** (e - 23)))
