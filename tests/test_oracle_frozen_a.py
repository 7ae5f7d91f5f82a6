"""Pins of the oracle's frozen-FP8-A path (the pages' training setup: A is
frozen and held in FP8, and X~ A~^T is formed in the forward for dL/dB).

  * U = X~ A~^T / (s_x s_a) against exact rationals on a tiny case, and against
    a scaled identity A~ (closed form);
  * dB of the frozen backward against central finite differences of the loss
    <G^, X^ (B DQ(A~))^T>, which is linear in B;
  * dB against the general backward with A = DQ(A~) (a differently written
    product: G^^T (X^ A^T) from fp32 A), up to the float32 store of U;
  * fp8_dequantize: exact decode at s = 1, exact rationals, and the E4M3
    quantize-dequantize error bound (half a step of the scaled value).
"""
from fractions import Fraction

import numpy as np

import oracle
from oracle import e4m3
from tests.exact import round_to_f32

DEC = e4m3.DECODE_F64


def rand_codes(rng, shape, hi=0x60):
    c = rng.integers(0, hi + 1, size=shape).astype(np.uint8)
    return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def tiny(seed, T=5, d_in=7, d_out=6, r=3):
    rng = np.random.default_rng(seed)
    return (rand_codes(rng, (T, d_in)), rand_codes(rng, (T, d_out)),
            rand_codes(rng, (d_out, d_in)), rand_codes(rng, (r, d_in)),
            rng.standard_normal((d_out, r)).astype(np.float32),
            np.float32(1.75), np.float32(0.3), np.float32(5.5), np.float32(96.0))


def test_u_exact_rationals_tiny():
    xq, gq, wq, aq, B, s_x, s_g, s_w, s_a = tiny(1)
    y, u = oracle.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a)
    assert u.shape == (xq.shape[0], aq.shape[0]) and u.dtype == np.float32
    assert np.array_equal(y, oracle.melded_linear_fwd(xq, s_x, wq, s_w))
    for t in range(u.shape[0]):
        for k in range(u.shape[1]):
            acc = sum(Fraction(DEC[xq[t, j]]) * Fraction(DEC[aq[k, j]])
                      for j in range(xq.shape[1]))
            ref = round_to_f32(acc / (Fraction(float(s_x)) * Fraction(float(s_a))))
            assert abs(u[t, k] - ref) <= abs(ref) * 2.0 ** -23


def test_u_scaled_identity():
    """A~ = c I on the first r inputs -> U[:, k] = dec(X~[:, k]) c / (s_x s_a)."""
    rng = np.random.default_rng(2)
    xq = rand_codes(rng, (9, 32))
    aq = np.zeros((4, 32), np.uint8)
    aq[np.arange(4), np.arange(4)] = 0x44                  # 3.0 = 1.5 * 2^1
    wq = rand_codes(rng, (16, 32))
    _, u = oracle.melded_linear_fwd_frozen_a(xq, 2.0, wq, 1.0, aq, 0.75)
    assert np.array_equal(u, (DEC[xq[:, :4]] * 3.0 / 1.5).astype(np.float32))


def test_frozen_db_matches_finite_differences():
    xq, gq, wq, aq, B, s_x, s_g, s_w, s_a = tiny(3)
    _, u = oracle.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a)
    _, dB = oracle.melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, u)
    g_hat = DEC[gq] / float(s_g)
    x_hat = DEC[xq] / float(s_x)
    a_hat = DEC[aq] / float(s_a)

    def L(Bm):              # <G^, X^ (B A^)^T>, explicit sums
        return sum(g_hat[t, o] * x_hat[t, j] * sum(Bm[o, k] * a_hat[k, j]
                                                   for k in range(Bm.shape[1]))
                   for t in range(g_hat.shape[0]) for o in range(g_hat.shape[1])
                   for j in range(x_hat.shape[1]))
    B64 = B.astype(np.float64)
    fd = np.zeros_like(B64)
    h = 1e-3
    for o in range(B.shape[0]):
        for k in range(B.shape[1]):
            p, m = B64.copy(), B64.copy()
            p[o, k] += h
            m[o, k] -= h
            fd[o, k] = (L(p) - L(m)) / (2 * h)
    # U is stored as float32: relative 2^-24 per element
    assert np.allclose(dB, fd, rtol=1e-6, atol=1e-6 * np.abs(fd).max())


def test_frozen_db_matches_general_backward():
    xq, gq, wq, aq, B, s_x, s_g, s_w, s_a = tiny(4, T=40, d_in=48, d_out=32, r=5)
    _, u = oracle.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a)
    dx_f, dB_f = oracle.melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, u)
    A = oracle.dequantize(aq, s_a)                     # float64, exact
    dx, _, dB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, want_da=False)
    assert np.array_equal(dx_f, dx)
    np.testing.assert_allclose(dB_f, dB, rtol=1e-6, atol=1e-6 * np.abs(dB).max())


def test_frozen_backward_no_tokens():
    xq, gq, wq, aq, B, s_x, s_g, s_w, s_a = tiny(5)
    _, u = oracle.melded_linear_fwd_frozen_a(xq[:0], s_x, wq, s_w, aq, s_a)
    dx, dB = oracle.melded_linear_bwd_frozen_a(gq[:0], s_g, wq, s_w, u)
    assert u.shape == (0, aq.shape[0]) and dx.shape == (0, wq.shape[1]) and not dB.any()


def test_dequantize_exact_and_error_bound():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                  # no NaN codes
    assert np.array_equal(oracle.fp8_dequantize(codes, 1.0), e4m3.DECODE_F32[codes])
    for s in (3.0, 0.1, 448.0 / 7.3):
        s32 = np.float32(s)
        dq = oracle.fp8_dequantize(codes, s32)
        for c, v in zip(codes[::7], dq[::7]):
            assert v == np.float32(round_to_f32(Fraction(float(DEC[c])) / Fraction(float(s32))))
    # quantize -> dequantize stays within half an E4M3 step of the scaled value
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(4000) * 0.02).astype(np.float32)
    q, s, _, _ = oracle.fp8_quantize(x)
    back = oracle.fp8_dequantize(q, s).astype(np.float64)
    v = x.astype(np.float64) * float(s)
    bound = e4m3.step_of(np.abs(v)) / 2 / float(s)
    assert np.all(np.abs(back - x) <= bound * (1 + 1e-6) + 1e-12)
