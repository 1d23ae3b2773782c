"""Write dequant_rounding.json: cases where the dequantisation's two binary32
roundings, fl(fl(acc * rs) * cs), differ from a single rounding of the exact
product acc * rs * cs.

Everything here is exact rational arithmetic with round-to-nearest-even to
binary32 written out below; it calls neither the oracle nor the GPU library.
The chosen accumulators are then written as dot products of int8 rows so a
test can feed them through a GEMM.

    python tests/golden/make_dequant_rounding.py
"""
import json
import os
import random
import struct
from fractions import Fraction


def round_binary32(x: Fraction) -> Fraction:
    """Nearest binary32 value to x (ties to even); normal range only."""
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
    if e < -126 or e > 127:
        raise ValueError("outside the normal binary32 range")
    scaled = a * (1 << 23)
    q = scaled.numerator // scaled.denominator
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return sign * Fraction(q, 1 << 23) * Fraction(2) ** e


def bits(v: Fraction) -> str:
    # v is exactly representable in binary32, hence in binary64: the
    # conversions below are exact
    return "0x%08x" % struct.unpack("<I", struct.pack("<f", float(v)))[0]


def int8_rows_for(acc: int):
    """int8 rows a, b (length 16) with sum(a*b) == acc."""
    sign = 1 if acc >= 0 else -1
    n = abs(acc)
    q, rem = divmod(n, 127 * 127)
    t, u = divmod(rem, 127)
    a = [127] * q + [127, u]
    b = [127] * q + [t, 1]
    assert len(a) <= 16 and all(-128 <= v <= 127 for v in a + b)
    a += [0] * (16 - len(a))
    b += [0] * (16 - len(b))
    b = [sign * v for v in b]
    assert sum(x * y for x, y in zip(a, b)) == acc
    return a, b


def main():
    rng = random.Random(5)
    cases = []
    while len(cases) < 3:
        acc = rng.randint(-300000, 300000)
        rs = round_binary32(Fraction(rng.randint(1000, 10000), 1000000))
        cs = round_binary32(Fraction(rng.randint(1000, 10000), 1000000))
        two = round_binary32(round_binary32(Fraction(acc) * rs) * cs)
        one = round_binary32(Fraction(acc) * rs * cs)
        if two != one:
            a, b = int8_rows_for(acc)
            cases.append({"acc": acc, "a_row": a, "b_col": b,
                          "row_scale_bits": bits(rs), "col_scale_bits": bits(cs),
                          "expected_bits": bits(two), "single_rounding_bits": bits(one)})
    out = {
        "about": ("Dequantisation out = ((float)acc * row_scale) * col_scale, each product "
                  "rounded to binary32 (nearest even), for accumulators where this differs "
                  "from rounding acc*rs*cs once; derived by exact rational arithmetic in "
                  "make_dequant_rounding.py.  acc = sum(a_row[k] * b_col[k])."),
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dequant_rounding.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
