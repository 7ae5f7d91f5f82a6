"""Exact-arithmetic helpers for the oracle's pins (no FP8 or method code here).

round_to_f32 rounds an exact rational to the nearest float32, ties to even,
written from the IEEE-754 binary32 definition; fmaf_exact(a, b, c) is then the
correctly rounded fused multiply-add, i.e. round_to_f32(a*b + c) computed on
exact rationals.  These let tests check the oracle's fmaf chain and fp32 steps
without trusting any floating-point library.
"""
from fractions import Fraction
import math

import numpy as np

F32_MAX = Fraction(2) ** 127 * (2 - Fraction(1, 2 ** 23))


def round_to_f32(x: Fraction) -> float:
    if x == 0:
        return 0.0
    neg = x < 0
    a = -x if neg else x
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 23)      # spacing of binary32 at a
    n = a / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v > F32_MAX:
        out = math.inf
    else:
        out = float(v)
    return -out if neg else out


def fmaf_exact(a: float, b: float, c: float) -> float:
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    r = round_to_f32(exact)
    if exact == 0:
        # exact zero sum: IEEE gives +0 in round-to-nearest unless both
        # addends are -0 (a*b and c both negative zero)
        prod_neg = (math.copysign(1.0, a) * math.copysign(1.0, b)) < 0
        prod_zero = (a == 0 or b == 0)
        if prod_zero and c == 0 and prod_neg and math.copysign(1.0, c) < 0:
            return -0.0
        return 0.0
    return r


def f32(x) -> float:
    return float(np.float32(x))
