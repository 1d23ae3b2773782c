"""Write quantize_ties.json: fp16 rows [amax, x] whose quantisation with
scale = fl32(amax / 127) puts x / scale exactly on a tie n + 1/2, where the
correctly rounded quotient keeps the tie (so q is the even neighbour) but
multiplying by the rounded reciprocal fl32(1 / scale) leaves it.

The search uses numpy float arithmetic only to find candidates; every stored
case is then re-derived with exact rational arithmetic and binary32 rounding
written out (tests/exact_binary32.py).  Neither the oracle nor the GPU
library is involved.

    python tests/golden/make_quantize_ties.py
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
from exact_binary32 import round_binary32, round_half_even  # noqa: E402


def main():
    amax = np.arange(0x0400, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float32)
    s = (amax / np.float32(127)).astype(np.float32)
    inv = (np.float32(1) / s).astype(np.float32)
    cases = []
    for n in range(0, 127):
        x = (n + 0.5) * s.astype(np.float64)
        ok = (x.astype(np.float16).astype(np.float64) == x) & (x <= amax.astype(np.float64))
        idx = np.nonzero(ok)[0]
        if idx.size == 0:
            continue
        t2 = (x[idx].astype(np.float32) * inv[idx]).astype(np.float32)
        for j in idx[np.rint(t2) != np.rint(np.float32(n + 0.5))]:
            a, xv = float(amax[j]), float(x[j])
            S = round_binary32(Fraction(a) / 127)
            q = round_half_even(round_binary32(Fraction(xv) / S))
            q_recip = round_half_even(round_binary32(Fraction(xv) * round_binary32(1 / S)))
            if q != q_recip:
                cases.append({"row_f16_bits": ["0x%04x" % int(np.float16(a).view(np.uint16)),
                                               "0x%04x" % int(np.float16(xv).view(np.uint16))],
                              "row_values": [a, xv], "expected_q": [127, q],
                              "reciprocal_multiply_q": [127, q_recip], "tie": n + 0.5})
                break
        if len(cases) >= 4:
            break
    out = {"about": ("Per-row int8 quantisation, scale = fl32(absmax / 127), q = nearest-even "
                     "integer to fl32(x / scale): rows where x / scale is exactly a tie and "
                     "the rounded-reciprocal shortcut would round the other way.  Derived by "
                     "exact rational arithmetic in make_quantize_ties.py."),
           "cases": cases}
    path = os.path.join(HERE, "quantize_ties.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path, len(cases))


if __name__ == "__main__":
    main()
