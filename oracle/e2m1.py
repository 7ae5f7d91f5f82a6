"""OCP FP4 E2M1 in software, written from the format's definition.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.

The FALQON pages mention FP4 only as an estimate (OpenReview rebuttal on
paperhub.cn, thread 2, point W2 and Table R3: the FP4 speed-up is estimated
from the FP4/FP8 matrix-multiplication throughput ratio); they define no FP4
format or recipe.  The format used here is the 4-bit element of the OCP
Microscaling specification, E2M1:

* 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
* exponent field 0 holds the subnormals 0 and 0.5;
* magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); no infinity, no NaN.

Encoding (reading used, the same conventions as the FP8 casts here): round
to the nearest representable value, ties to the even code (mantissa bit 0);
finite overflow and infinities saturate to +-6; NaN, which has no encoding,
becomes zero with the input's sign bit.  The sign of zero is kept.

Packing (reading used): two codes per byte, the element with the lower
index in the low nibble.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0


def decode_code(c: int) -> float:
    """Value of one E2M1 code 0..15 (a Python float, exact)."""
    s = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:
        return s * m * 0.5
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


#: decode table, float64, index = code (16 entries)
DECODE_F64 = np.array([decode_code(c) for c in range(16)], dtype=np.float64)


def decode(q: np.ndarray) -> np.ndarray:
    """Codes (integer array of values 0..15) -> float64 values, exactly."""
    return DECODE_F64[np.asarray(q, dtype=np.uint8) & 0xF]


def encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> E2M1 codes (uint8 0..15): round to nearest, ties to
    even, saturate, NaN to a signed zero.

    For a = |v|: the grid spacing is 0.5 below 2 and 2**(floor(log2 a) - 1)
    above; n = a / spacing rounded to the nearest integer (ties to even), and
    the code is that of n * spacing, clamped to the largest magnitude.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    sign = ((v.view(np.uint32) >> 31).astype(np.uint8) << 3).astype(np.uint8)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, np.abs(v.astype(np.float64)))
    a = np.minimum(a, 8.0)                        # everything above 6 saturates anyway
    _, e = np.frexp(np.where(a < 2.0, 1.0, a))    # a = f * 2**e, f in [0.5, 1)
    spacing = np.where(a < 2.0, 0.5, np.ldexp(1.0, e - 2))
    val = np.rint(a / spacing) * spacing          # rint: half to even
    val = np.minimum(val, E2M1_MAX)
    code = np.searchsorted(DECODE_F64[:8], val)   # val is one of the 8 magnitudes
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def pack(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] codes -> [..., n] bytes, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack(b: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] codes."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out
