"""Pins of the oracle's FP4 E2M1 encoding, quantize and forward product.

  * the decode table has the structure of a 1-2-1 binary format with
    exponent bias 1 (sign symmetry, two values per binade with the spacing
    halving per binade downwards, largest magnitude 6, smallest 0.5), and
    every value is exact in E4M3 and in bfloat16;
  * the encoder equals a brute-force nearest-value search over the eight
    magnitudes (ties to the code with mantissa bit 0) on a dense sweep and on
    random values; the ties are listed as exact rationals;
  * infinities saturate, NaN gives a signed zero, the sign of zero is kept;
  * two codes per byte, the lower index in the low nibble;
  * fp4_quantize: the largest element maps to +-6, quantizing the dequantized
    tensor again gives the same codes;
  * the FP4 forward product equals an integer matrix product of the doubled
    code values, divided by 4 s_x s_w.
"""
import numpy as np

import oracle
from oracle import e2m1, e4m3


def brute_encode(v):
    """Nearest E2M1 magnitude by exhaustive search; ties to the even code."""
    v = np.asarray(v, dtype=np.float32)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(v):
        a = abs(float(x))
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        code = best[0] if best.size == 1 else [c for c in best if c % 2 == 0][0]
        out[idx] = code | (8 if np.signbit(x) else 0)
    return out


def test_decode_table_structure():
    t = e2m1.DECODE_F64
    assert t.shape == (16,)
    assert np.array_equal(t[8:], -t[:8]) and np.signbit(t[8]) and not np.signbit(t[0])
    pos = t[:8]
    assert np.all(np.diff(pos) > 0) and pos[0] == 0 and pos[1] == 0.5 and pos[7] == 6.0
    # binades [1,2), [2,4), [4,8) hold two values each, spacing 2**(k-1)
    for k, (lo, hi) in enumerate([(2, 4), (4, 6), (6, 8)]):
        assert pos[lo] == 2.0 ** k and pos[lo + 1] - pos[lo] == 2.0 ** (k - 1)
    # exact in E4M3 and in bfloat16
    assert np.array_equal(e4m3.decode(e4m3.encode(t.astype(np.float32))), t)
    bf = (t.astype(np.float32).view(np.uint32) >> 16 << 16).view(np.float32)
    assert np.array_equal(bf.astype(np.float64), t)


def test_encode_matches_brute_force():
    grid = np.arange(-8 * 256, 8 * 256 + 1, dtype=np.float64) / 256.0
    rng = np.random.default_rng(3)
    rnd = np.concatenate([rng.standard_normal(4000) * 3.0, rng.uniform(-7, 7, 4000),
                          rng.standard_normal(500) * 1e-3, rng.standard_normal(500) * 1e4])
    v = np.concatenate([grid, rnd]).astype(np.float32)
    assert np.array_equal(e2m1.encode(v), brute_encode(v))


def test_ties_to_even_and_specials():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in ties.items():
        for sgn in (1.0, -1.0):
            got = e2m1.decode(e2m1.encode(np.array([sgn * x], np.float32)))[0]
            assert got == sgn * want, (sgn * x, got)
    v = np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, 6.0, 7.0, 1e30, -1e30], np.float32)
    c = e2m1.encode(v)
    assert list(c[:2]) == [0x7, 0xF]
    assert e2m1.decode(c[2:4]).tolist() == [0.0, 0.0] and (c[2] & 7) == 0 and (c[3] & 7) == 0
    assert list(c[4:6]) == [0x0, 0x8]
    assert list(c[6:]) == [0x7, 0x7, 0x7, 0xF]


def test_pack_order_and_roundtrip():
    assert e2m1.pack(np.array([1, 2], np.uint8)).tolist() == [0x21]
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, size=(7, 24)).astype(np.uint8)
    assert np.array_equal(e2m1.unpack(e2m1.pack(c)), c)


def test_fp4_quantize_amax_and_idempotence():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((33, 64)) * 3.0).astype(np.float32)
    x[5, 7] = -40.0
    q, s, amax, bad = oracle.fp4_quantize(x)
    assert amax == 40.0 and bad == 0 and s == np.float32(6.0) / np.float32(40.0)
    codes = e2m1.unpack(q)
    assert codes[5, 7] == 0xF and np.all(np.abs(e2m1.decode(codes)) <= 6.0)
    # dequantize (exactly representable multiples) and quantize again with s
    xd = (e2m1.decode(codes) / np.float64(s)).astype(np.float32)
    q2, _, _, _ = oracle.fp4_quantize(xd, scale_in=float(s))
    assert np.array_equal(q2, q)
    # non-finite inputs are counted and excluded from amax
    x[0, 0] = np.nan
    x[1, 1] = np.inf
    q3, s3, amax3, bad3 = oracle.fp4_quantize(x)
    assert bad3 == 2 and amax3 == 40.0
    assert e2m1.unpack(q3)[1, 1] == 0x7 and (e2m1.unpack(q3)[0, 0] & 7) == 0


def test_fp4_forward_is_an_exact_integer_product():
    rng = np.random.default_rng(6)
    T, d_in, d_out = 9, 64, 11
    xq = e2m1.pack(rng.integers(0, 16, size=(T, d_in)).astype(np.uint8))
    wq = e2m1.pack(rng.integers(0, 16, size=(d_out, d_in)).astype(np.uint8))
    s_x, s_w = np.float32(0.37), np.float32(5.5)
    y = oracle.melded_linear_fwd_fp4(xq, s_x, wq, s_w)
    twice = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4, 5: 6, 6: 8, 7: 12}
    xi = np.vectorize(lambda c: (-1 if c & 8 else 1) * twice[c & 7])(e2m1.unpack(xq)).astype(np.int64)
    wi = np.vectorize(lambda c: (-1 if c & 8 else 1) * twice[c & 7])(e2m1.unpack(wq)).astype(np.int64)
    ref = ((xi @ wi.T).astype(np.float64) / (4.0 * np.float64(s_x) * np.float64(s_w))).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
