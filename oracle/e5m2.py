"""OCP FP8 E5M2 in software, written from the format's definition.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.

The FALQON pages name the FP8 formats only as "E4M3 or E5M2" (OpenReview
rebuttal on paperhub.cn, thread 2, point W2).  E5M2 serves here as the
optional format of the upstream gradient dY.  Bit layout (OCP 8-bit floating
point specification, E5M2):

* 1 sign bit, 5 exponent bits (bias 15), 2 mantissa bits;
* exponent field 0 holds the subnormals m * 2**-16, m = 0..3;
* exponent field 31: S.11111.00 is infinity, S.11111.{01,10,11} are NaN;
* largest finite magnitude 57344 = 1.75 * 2**15 (0x7B), smallest normal
  2**-14 (0x04).

Encoding rounds to the nearest representable value, ties to the even code,
and saturates finite overflow and infinities to +-57344 (the same saturating
convention as the E4M3 casts here).  The sign is kept (-0.0 -> 0x80).  NaN
encodes to 0x7F with the input's sign bit.
"""
from __future__ import annotations

import numpy as np

E5M2_MAX = 57344.0
MIN_NORMAL = 2.0 ** -14
SUBNORMAL_STEP = 2.0 ** -16


def decode_code(c: int) -> float:
    """Value of one E5M2 code (a Python float, exact)."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 2) & 0x1F
    m = c & 0x3
    if e == 0x1F:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * m * SUBNORMAL_STEP
    return s * (1.0 + m / 4.0) * 2.0 ** (e - 15)


#: decode table, float64, index = code (256 entries; +-inf at 0x7C / 0xFC)
DECODE_F64 = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
#: the same table in float32 (every E5M2 value is exact in float32)
DECODE_F32 = DECODE_F64.astype(np.float32)


def decode(q: np.ndarray) -> np.ndarray:
    """Codes (uint8 array) -> float64 values, exactly."""
    return DECODE_F64[np.asarray(q, dtype=np.uint8)]


def encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> E5M2 codes: round to nearest, ties to even, saturate.

    For the magnitude a = |v| (the sign bit is put back at the end):
      1. NaN -> 0x7F; a >= 57344 (including +inf) -> 0x7B;
      2. the grid spacing at a: 2**-16 below 2**-14, else 2**(floor(log2 a) - 2);
      3. n = a / spacing rounded to the nearest integer, ties to even;
      4. the code of n * spacing (a carry into the next binade, or past the
         largest value, is absorbed by the code arithmetic and the clamp).
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    bits = v.view(np.uint32)
    sign = ((bits >> 31).astype(np.uint8) << 7).astype(np.uint8)
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(v)
    sat = np.zeros(v.shape, dtype=bool)
    np.greater_equal(a, E5M2_MAX, out=sat, where=~nan)
    a_ok = np.where(nan | sat, 0.0, a)

    _, e = np.frexp(a_ok)                      # a = f * 2**e, f in [0.5, 1)
    spacing = np.where(a_ok < MIN_NORMAL, SUBNORMAL_STEP, np.ldexp(1.0, e - 1 - 2))
    n = np.rint(a_ok / spacing)                # round half to even
    val = n * spacing                          # at most 4 significant bits

    sub = val < MIN_NORMAL
    code_sub = np.rint(val / SUBNORMAL_STEP)
    vn = np.where(sub, 1.0, val)
    _, e2 = np.frexp(vn)
    ex = e2 - 1                                # floor(log2 val)
    mant = np.rint((vn / np.ldexp(1.0, ex) - 1.0) * 4.0)
    code_norm = (ex + 15) * 4 + mant
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.minimum(code, 0x7B)              # a value rounded up to 2**16 saturates
    code = np.where(sat, 0x7B, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def step_of(m: np.ndarray) -> np.ndarray:
    """Spacing of the E5M2 grid at magnitude m >= 0 (float64):
    2**(floor(log2 m) - 2) for m >= 2**-14, else 2**-16."""
    m = np.asarray(m, dtype=np.float64)
    _, e = np.frexp(np.where(m < MIN_NORMAL, 1.0, m))
    return np.where(m < MIN_NORMAL, SUBNORMAL_STEP, np.ldexp(1.0, e - 1 - 2))
