"""Exact rounding of rationals to IEEE binary32 (nearest, ties to even),
written out for tests that derive expected values independently of any
floating-point library."""
from fractions import Fraction


def round_binary32(x: Fraction) -> Fraction:
    """Nearest binary32 value to x, ties to even (normal and subnormal range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    if e > 127:
        raise OverflowError("outside the binary32 range")
    # 24 significant bits for normals; subnormals keep bits down to 2^-149
    frac_bits = 23 if e >= -126 else 23 - (-126 - e)
    scaled = a * Fraction(2) ** frac_bits
    q = scaled.numerator // scaled.denominator
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return sign * Fraction(q) / Fraction(2) ** frac_bits * Fraction(2) ** e


def round_half_even(x: Fraction) -> int:
    q = x.numerator // x.denominator   # floor
    rem = x - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return q
