"""Writes fp8_double_rounding.txt: inputs on which the quantize's two
roundings (fl32(x * s), then E4M3 nearest-even) give another code than one
rounding of the exact product x * s would.

The quantize multiplies by the per-tensor scale and rounds the product to
FP8 (FALQON OpenReview rebuttal on paperhub.cn, thread 2, reply W2); the page
does not say whether the product is first rounded to float32, and the reading
taken is that it is (an fp32 multiply, then the cast).  A float32 rounding
cannot carry a value across an E4M3 midpoint (the midpoints are float32
values and rounding is monotone), so the two readings differ exactly when
fl32(x * s) lands ON a midpoint that x * s itself misses by less than half a
float32 spacing: the tie then goes to the even code, while the exact product
goes to the code on its own side.

Everything here is exact rational arithmetic (fractions.Fraction) on the
E4M3 values as the OCP 8-bit floating-point specification defines them
(bias 7, three mantissa bits, subnormals m * 2^-9, largest finite 448); no
code of the oracle or of the GPU library is used.  Run from the repository
root:  python tests/golden/make_fp8_double_rounding.py
"""
from __future__ import annotations

import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from tests.exact import round_to_f32  # noqa: E402

# the 127 non-negative finite E4M3 values and their codes
VALUES = []
for code in range(0x7F):
    e, m = code >> 3, code & 7
    v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    VALUES.append((v, code))


def e4m3_nearest(v: Fraction) -> int:
    """Code of the E4M3 value nearest to v, ties to the even code, magnitudes
    past 448 saturated, the sign bit kept."""
    sign = 0x80 if v < 0 else 0
    a = abs(v)
    if a >= 448:
        return 0x7E | sign
    best = min(VALUES, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return best[1] | sign


def f32(x: float) -> float:
    assert float(np.float32(x)) == x, x
    return x


def search(s: float, mid: Fraction, above: bool):
    """A float32 x near mid / s whose exact product with s misses `mid` on the
    requested side by less than half the float32 spacing at mid."""
    x0 = np.float32(float(mid) / s)
    for k in range(-64, 65):
        x = x0
        step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
        for _ in range(abs(k)):
            x = np.nextafter(x, step)
        p = Fraction(float(x)) * Fraction(s)
        if p == mid or (p > mid) != above:
            continue
        if Fraction(round_to_f32(p)) == mid:
            return float(x)
    return None


def main():
    # midpoints between neighbouring E4M3 values (a, code_a) < (b, code_b);
    # the tie goes to the even code
    mids = [(Fraction(1, 1024), 0x00, 0x01),          # 2^-10: between 0 and 2^-9
            (Fraction(17, 16), 0x38, 0x39),           # 1.0625: between 1 and 1.125
            (Fraction(19, 16), 0x39, 0x3A),           # 1.1875: between 1.125 and 1.25
            (Fraction(25, 4), 0x4C, 0x4D),            # 6.25: between 6 and 6.5
            (Fraction(432), 0x7D, 0x7E),              # between 416 and 448
            (Fraction(15, 1024), 0x07, 0x08)]         # between 7*2^-9 and 2^-6
    rows = []
    scales = [f32(float(np.float32(448.0) / np.float32(3.1))),     # current scaling, amax 3.1
              f32(float(np.float32(448.0) / np.float32(0.0731))),  # amax 0.0731
              f32(float(np.float32(1.7))), f32(float(np.float32(0.3)))]
    for mid, ca, cb in mids:
        va = dict((c, v) for v, c in VALUES)[ca]
        vb = dict((c, v) for v, c in VALUES)[cb]
        assert va < mid < vb and mid == (va + vb) / 2, (mid, ca, cb)
        even = ca if ca % 2 == 0 else cb
        for s in scales:
            for above in (True, False):
                # the side whose single rounding is NOT the even code
                if (above and even == cb) or (not above and even == ca):
                    continue
                x = search(s, mid, above)
                if x is None:
                    continue
                for sign in (1, -1):
                    xs = sign * x
                    p = Fraction(xs) * Fraction(s)
                    two = e4m3_nearest(Fraction(round_to_f32(p)))
                    one = e4m3_nearest(p)
                    assert two != one
                    rows.append((xs, s, two, one, sign * mid, ca, cb))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_double_rounding.txt")
    with open(out, "w") as fh:
        fh.write("# Written by tests/golden/make_fp8_double_rounding.py (exact rationals; see its\n"
                 "# docstring).  x and s are float32 values (hex floats); fl32(x*s) is the E4M3\n"
                 "# midpoint `mid` between the codes lo and hi, while the exact x*s misses it.\n"
                 "# code2 = E4M3(fl32(x*s)) (the tie goes to the even code), code1 = E4M3 of the\n"
                 "# exact product (one rounding).\n")
        fh.write("# x s code2 code1 mid lo hi\n")
        for xs, s, two, one, mid, ca, cb in rows:
            fh.write(f"{float(xs).hex()} {float(s).hex()} 0x{two:02X} 0x{one:02X} "
                     f"{float(mid)!r} 0x{ca:02X} 0x{cb:02X}\n")
    print(f"wrote {len(rows)} cases to {out}")


if __name__ == "__main__":
    main()
