"""OCP FP8 E4M3 ("e4m3fn") in software, written from the format's definition.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.

The FALQON pages name the FP8 formats only as "E4M3 or E5M2" (OpenReview
rebuttal on paperhub.cn, reply to reviewer 2, point W2).  The bit layout used
here is the OCP 8-bit floating-point specification's E4M3:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 holds the subnormals m * 2**-9, m = 0..7;
* no infinities; S.1111.111 (0x7F / 0xFF) is NaN;
* largest finite magnitude 448 (0x7E), smallest normal 2**-6 (0x08).

Encoding rounds to the nearest representable value, ties to the even code
(the code whose last bit is 0), and saturates finite overflow and infinities
to +-448.  The sign is kept, so -0.0 encodes to 0x80.  NaN encodes to 0x7F
with the input's sign bit.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP = 2.0 ** -9


def decode_code(c: int) -> float:
    """Value of one E4M3 code (a Python float, exact)."""
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * SUBNORMAL_STEP
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: decode table, float64, index = code (256 entries; NaN at 0x7F and 0xFF)
DECODE_F64 = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
#: the same table in float32 (every E4M3 value is exact in float32)
DECODE_F32 = DECODE_F64.astype(np.float32)


def decode(q: np.ndarray) -> np.ndarray:
    """Codes (uint8 array) -> float64 values, exactly."""
    return DECODE_F64[np.asarray(q, dtype=np.uint8)]


def decode_f32(q: np.ndarray) -> np.ndarray:
    return DECODE_F32[np.asarray(q, dtype=np.uint8)]


def encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3 codes: round to nearest, ties to even, saturate.

    Steps, for the magnitude a = |v| (the sign bit is put back at the end):
      1. NaN -> 0x7F; a >= 448 (including +inf) -> 0x7E.
      2. the grid spacing at a: 2**-9 below 2**-6, else 2**(floor(log2 a) - 3);
      3. n = a / spacing rounded to the nearest integer, ties to even (the
         parity of n is the parity of the code's last bit);
      4. the code of the value n * spacing.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    bits = v.view(np.uint32)
    sign = ((bits >> 31).astype(np.uint8) << 7).astype(np.uint8)
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(v)
    sat = np.zeros(v.shape, dtype=bool)
    np.greater_equal(a, E4M3_MAX, out=sat, where=~nan)
    a_ok = np.where(nan | sat, 0.0, a)

    _, e = np.frexp(a_ok)                      # a = f * 2**e, f in [0.5, 1)
    spacing = np.where(a_ok < MIN_NORMAL, SUBNORMAL_STEP, np.ldexp(1.0, e - 1 - 3))
    n = np.rint(a_ok / spacing)                # round half to even
    val = n * spacing                          # exact: at most 5 significant bits

    # code of val
    sub = val < MIN_NORMAL
    code_sub = np.rint(val / SUBNORMAL_STEP)
    vn = np.where(sub, 1.0, val)
    _, e2 = np.frexp(vn)
    ex = e2 - 1                                # floor(log2 val)
    mant = np.rint((vn / np.ldexp(1.0, ex) - 1.0) * 8.0)
    code_norm = (ex + 7) * 8 + mant
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def step_of(m: np.ndarray) -> np.ndarray:
    """Spacing of the E4M3 grid at magnitude m >= 0 (float64):
    2**(floor(log2 m) - 3) for m >= 2**-6, else 2**-9 (this includes m == 0)."""
    m = np.asarray(m, dtype=np.float64)
    _, e = np.frexp(np.where(m < MIN_NORMAL, 1.0, m))
    return np.where(m < MIN_NORMAL, SUBNORMAL_STEP, np.ldexp(1.0, e - 1 - 3))
