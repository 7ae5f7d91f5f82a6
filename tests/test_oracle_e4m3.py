"""Pins of the oracle's E4M3 format code against definitions it does not use.

* decode: every code against PyTorch's own float8_e4m3fn type (a library
  routine written by others) and against landmark values of the format;
* encode: against a brute-force nearest-value search over the 127 finite
  magnitudes (ties to the even code, saturation at 448), over a structured set
  of ~6 million float32 bit patterns that holds every rounding tie and the
  values one float32 step either side of each tie, plus random patterns; and
  against PyTorch's cast inside the range where PyTorch does not saturate;
* Q(DQ(q)) == q for every non-NaN code.
"""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_for_all_256_codes():
    ref = torch_decode_all()
    ours = e4m3.DECODE_F64
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    # signs of zero too
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(ours[~nan_ref]))


def test_decode_landmarks():
    d = e4m3.DECODE_F64
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x01] == 2.0 ** -9
    assert d[0x07] == 7 * 2.0 ** -9
    assert d[0x08] == 2.0 ** -6
    assert d[0x38] == 1.0
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    # closed form (-1)^s 2^(e-7) (1 + m/8), subnormal (-1)^s 2^-6 m/8
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (2.0 ** -6) * (m / 8) if e == 0 else (2.0 ** (e - 7)) * (1 + m / 8)
        assert d[c] == (-v if s else v)


def brute_force_encode(v: np.ndarray) -> np.ndarray:
    """Nearest of the 127 non-negative finite E4M3 magnitudes (PyTorch's decode
    table), ties to the even code, saturating; sign copied; NaN -> 0x7F|sign."""
    mags = torch_decode_all()[:127]               # codes 0..126, increasing
    assert np.all(np.diff(mags) > 0)
    v = np.asarray(v, np.float32)
    nan = np.isnan(v)
    a0 = np.where(nan, 0.0, np.abs(v.astype(np.float64)))
    hi = np.clip(np.searchsorted(mags, a0, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = np.abs(a0 - mags[lo])
    dhi = np.abs(mags[hi] - a0)
    pick = np.where(dlo < dhi, lo, hi)
    tie = dlo == dhi
    pick = np.where(tie & (lo != hi), np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a0 >= 448.0, 126, pick)
    code = pick.astype(np.uint8)
    code = np.where(nan, 0x7F, code).astype(np.uint8)
    sign = ((v.view(np.uint32) >> 31).astype(np.uint8) << 7).astype(np.uint8)
    return code | sign


def structured_f32_patterns():
    top = np.arange(1 << 20, dtype=np.uint32) << 12           # every sign/exponent/top-8 mantissa
    lows = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    pats = (top[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(12345)
    rnd = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd]).view(np.float32)


def test_encode_matches_brute_force_structured():
    v = structured_f32_patterns()
    ours = e4m3.encode(v)
    ref = brute_force_encode(v)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[:5]]} -> {ours[bad[:5]]} vs {ref[bad[:5]]}"


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-463.99, 463.99, 500_000),
        rng.standard_normal(500_000) * 0.01,
        rng.standard_normal(200_000) * 2.0 ** -8,
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v), ref)


def load_landmarks():
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_landmarks.txt")
    rows = []
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        v, c = line.split()[:2]
        rows.append((float(v), int(c, 16)))
    return rows


def test_encode_hand_derived_landmarks():
    """tests/golden/e4m3_landmarks.txt: values derived by hand from the format."""
    rows = load_landmarks()
    assert len(rows) >= 15
    for x, c in rows:
        assert e4m3.encode(np.array([x], np.float32))[0] == c, x
        assert brute_force_encode(np.array([x], np.float32))[0] == c, x


def test_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 1e30, np.inf, -np.inf, -1e30, 0.0, -0.0], np.float32)
    assert list(e4m3.encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80]
    n = e4m3.encode(np.array([np.nan, -np.nan], np.float32))
    assert n[0] & 0x7F == 0x7F and n[1] & 0x7F == 0x7F


@pytest.mark.parametrize("s", [1.0, 0.25, 1024.0, 3.7, 448.0 / 5.3, 1e-3])
def test_quantize_of_dequantize_is_identity(s):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    s32 = np.float32(s)
    x = (e4m3.DECODE_F32[codes] / s32).astype(np.float32)       # DQ
    v = (x * s32).astype(np.float32)                             # scale back
    assert np.array_equal(e4m3.encode(v), codes)


def test_step_of():
    assert e4m3.step_of(np.array([0.0]))[0] == 2.0 ** -9
    assert e4m3.step_of(np.array([2.0 ** -7]))[0] == 2.0 ** -9
    assert e4m3.step_of(np.array([2.0 ** -6]))[0] == 2.0 ** -9
    assert e4m3.step_of(np.array([1.0]))[0] == 0.125
    assert e4m3.step_of(np.array([448.0]))[0] == 32.0
    # the step equals the distance to the next code up, for every normal code
    for c in range(0x08, 0x7E):
        assert e4m3.step_of(np.array([e4m3.DECODE_F64[c]]))[0] == \
            e4m3.DECODE_F64[c + 1] - e4m3.DECODE_F64[c]
