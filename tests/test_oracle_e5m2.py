"""Pins of the oracle's E5M2 format (OCP 8-bit floating point, E5M2), used for
the optional E5M2 upstream gradient.

E5M2 has binary16's sign and exponent fields (5 bits, bias 15): an E5M2 code c
is the float16 whose bit pattern is c << 8.  numpy's float16 (an independent
implementation of IEEE binary16) therefore decodes every code, and brute
force over the 256 codes checks the rounding.
"""
from fractions import Fraction

import numpy as np

import oracle
from oracle import e5m2

ALL = np.arange(256, dtype=np.uint16)


def f16_of_code(c):
    return (np.asarray(c, np.uint16) << 8).view(np.float16).astype(np.float64)


def test_decode_equals_binary16_top_byte():
    ref = f16_of_code(ALL)
    got = e5m2.DECODE_F64
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7B] == 57344.0 and got[0x04] == 2.0 ** -14 and got[0x01] == 2.0 ** -16
    assert got[0x7C] == np.inf and got[0xFC] == -np.inf


def finite_codes():
    v = e5m2.DECODE_F64
    return np.array([c for c in range(256) if np.isfinite(v[c])], dtype=np.uint8)


def test_round_trip_of_every_finite_code():
    c = finite_codes()
    assert np.array_equal(e5m2.encode(e5m2.DECODE_F32[c]), c)


def test_encode_is_nearest_ties_to_even_brute_force():
    codes = finite_codes()
    vals = e5m2.DECODE_F64[codes]
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.uniform(-6, 4.7, 4000),
        # midpoints between neighbours (ties) and their float32 neighbours
        (np.sort(np.unique(vals))[1:] + np.sort(np.unique(vals))[:-1]) / 2,
    ]).astype(np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))])
    x = x[np.abs(x) < 57344.0]
    got = e5m2.encode(x)
    for xi, ci in zip(x, got):
        d = np.abs(vals - float(xi))
        best = codes[d == d.min()]
        best = best[(np.signbit(e5m2.DECODE_F64[best]) == np.signbit(xi)) | (d.min() > 0)]
        if best.size > 1:                      # tie: the even code
            best = best[(best & 1) == 0]
        assert ci in best, (xi, hex(ci), [hex(b) for b in best])


def test_saturation_nan_and_signed_zero():
    x = np.array([57344, 60000, 1e9, np.inf, -np.inf, -60000, np.nan, -np.nan, 0.0, -0.0],
                 np.float32)
    c = e5m2.encode(x)
    assert list(c[:6]) == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB]
    assert c[6] & 0x7F == 0x7F and c[7] & 0x7F == 0x7F
    assert c[8] == 0x00 and c[9] == 0x80


def test_quantize_e5m2_amax_maps_to_max():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(3000) * 1e-3).astype(np.float32)
    q, s, amax, bad = oracle.fp8_quantize(x, fmt="e5m2")
    assert bad == 0 and amax == np.max(np.abs(x))
    assert s == np.float32(57344.0) / amax
    i = int(np.argmax(np.abs(x)))
    assert q[i] & 0x7F == 0x7B
    # quantize -> dequantize within half an E5M2 step of the scaled value
    v = x.astype(np.float64) * float(s)
    back = e5m2.decode(q)
    assert np.all(np.abs(back - v) <= e5m2.step_of(np.abs(v)) / 2 * (1 + 1e-6) + 1e-12)


def test_backward_with_e5m2_gradient_exact_rationals():
    rng = np.random.default_rng(3)
    T, d_in, d_out, r = 4, 6, 5, 2
    gq = rng.integers(0, 0x7B, (T, d_out)).astype(np.uint8) | \
        (rng.integers(0, 2, (T, d_out)).astype(np.uint8) << 7)
    xq = rng.integers(0, 0x60, (T, d_in)).astype(np.uint8)
    wq = rng.integers(0, 0x60, (d_out, d_in)).astype(np.uint8)
    A = rng.standard_normal((r, d_in)).astype(np.float32)
    B = rng.standard_normal((d_out, r)).astype(np.float32)
    s_g, s_x, s_w = np.float32(3e4), np.float32(1.5), np.float32(7.0)
    dx, dA, dB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, g_fmt="e5m2")
    g = f16_of_code(gq)                        # decoded through binary16
    w = oracle.e4m3.decode(wq)
    for t in range(T):
        for k in range(d_in):
            acc = sum(Fraction(g[t, o]) * Fraction(w[o, k]) for o in range(d_out))
            ref = float(acc / (Fraction(float(s_g)) * Fraction(float(s_w))))
            assert abs(dx[t, k] - ref) <= abs(ref) * 2.0 ** -23
    g_hat = g / float(s_g)
    x_hat = oracle.e4m3.decode(xq) / float(s_x)
    np.testing.assert_allclose(dB, g_hat.T @ (x_hat @ A.astype(np.float64).T), rtol=1e-6)
    np.testing.assert_allclose(dA, (g_hat @ B.astype(np.float64)).T @ x_hat, rtol=1e-6)


def test_encode_matches_torch_cast_in_range():
    """torch's float8_e5m2 cast (round to nearest even) agrees wherever it does
    not overflow (it does not saturate: past 57344 it gives infinity)."""
    import torch
    from tests.test_oracle_e4m3 import structured_f32_patterns
    rng = np.random.default_rng(7)
    v = np.concatenate([
        structured_f32_patterns(),
        rng.uniform(-57343.0, 57343.0, 300_000).astype(np.float32),
        (rng.standard_normal(300_000) * 2.0 ** -14).astype(np.float32),
    ])
    with np.errstate(invalid="ignore"):
        v = v[np.isfinite(v) & (np.abs(v) <= 57344.0)]
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    ours = e5m2.encode(v)
    nan = np.isnan(v)
    bad = np.nonzero((ours != ref) & ~nan)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[:5]]} {ours[bad[:5]]} {ref[bad[:5]]}"
