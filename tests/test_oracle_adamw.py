"""Pins of the oracle's 32-bit AdamW adapter step (FALQON rebuttal on
paperhub.cn, thread 3 reply W3.1: the runs train with 32-bit AdamW).

The oracle fixes an fp32 operation order; these tests tie it to things other
than itself:
  * torch.optim.AdamW (an independent implementation of the published
    algorithm) run in float64 on the same inputs, over several steps;
  * closed forms of Adam: the first step moves every weight by lr * g / (|g| + eps)
    (sign descent), a constant gradient keeps that step size at every step,
    and with a zero gradient only the decoupled decay p * (1 - lr * wd) acts;
  * exact rational arithmetic for each rounding of one element.
A plausible mistake (no bias correction, eps inside the square root, L2 decay
added to the gradient, moments swapped) changes one of these by far more than
fp32 rounding.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
from tests.exact import round_to_f32

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def run_oracle(p, grads, hp=HP):
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    out = []
    for t, g in enumerate(grads, start=1):
        sc = oracle.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                  hp["weight_decay"], t)
        p, m, v = oracle.adamw_update(p, g, m, v, sc)
        out.append((p, m, v))
    return out


def run_torch(p, grads, hp=HP, cls=torch.optim.AdamW):
    """torch in float64, given the float32 values of the hyper-parameters (the
    C call takes them as float32)."""
    hp = {k: float(np.float32(x)) for k, x in hp.items()}
    w = torch.nn.Parameter(torch.tensor(p, dtype=torch.float64))
    opt = cls([w], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
              weight_decay=hp["weight_decay"], foreach=False)
    out = []
    for g in grads:
        w.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        st = opt.state[w]
        out.append((w.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
                     st["exp_avg_sq"].numpy().copy()))
    return out


def problem(seed, shape=(37, 19), steps=5):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(shape) * 0.05).astype(np.float32)
    grads = [(rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 0, shape)).astype(np.float32)
             for _ in range(steps)]
    return p, grads


@pytest.mark.parametrize("wd", [0.0, 0.01, 0.1])
def test_matches_torch_adamw_float64(wd):
    hp = dict(HP, weight_decay=wd)
    p0, grads = problem(1)
    ours = run_oracle(p0, grads, hp)
    ref = run_torch(p0, grads, hp)
    prev = p0.astype(np.float64)
    prev_ref = p0.astype(np.float64)
    for (p, m, v), (rp, rm, rv) in zip(ours, ref):
        # fp32 roundings, amplified where b1*m and (1-b1)*g nearly cancel
        np.testing.assert_allclose(m, rm, rtol=2e-5, atol=1e-6 * np.max(np.abs(rm)))
        np.testing.assert_allclose(v, rv, rtol=2e-5, atol=0)
        # compare the step itself (~lr), to the fp32 spacing of the weights
        np.testing.assert_allclose(p.astype(np.float64) - prev, rp - prev_ref,
                                   rtol=1e-4, atol=1e-8)   # fp32 ulp of |p| ~ 0.1
        prev, prev_ref = p.astype(np.float64), rp


def test_coupled_l2_decay_is_not_adamw():
    """torch.optim.Adam adds wd * p to the gradient (L2); the oracle must not."""
    p0, grads = problem(2)
    ours = run_oracle(p0, grads[:1], dict(HP, weight_decay=0.5))
    l2 = run_torch(p0, grads[:1], dict(HP, weight_decay=0.5), cls=torch.optim.Adam)
    assert np.max(np.abs(ours[0][0] - l2[0][0])) > 1e-5


def test_first_step_is_sign_descent():
    """Step 1: m^ = g and v^ = g^2, so p' = p - lr * g / (|g| + eps)."""
    rng = np.random.default_rng(3)
    p = rng.standard_normal(500).astype(np.float32)
    g = (rng.standard_normal(500) * 10.0 ** rng.uniform(-3, 2, 500)).astype(np.float32)
    (p1, m1, v1), = run_oracle(p, [g], dict(HP, weight_decay=0.0))
    expect = p.astype(np.float64) - 1e-3 * g / (np.abs(g.astype(np.float64)) + 1e-8)
    step, want = p1 - p.astype(np.float64), expect - p
    # fp32 roundings: relative on the step, plus one spacing of the weight
    assert np.all(np.abs(step - want) <= 1e-5 * np.abs(want) + np.spacing(np.abs(p)))
    np.testing.assert_allclose(m1, 0.1 * g.astype(np.float64), rtol=1e-6)
    np.testing.assert_allclose(v1, 0.001 * g.astype(np.float64) ** 2, rtol=2e-5)


def test_constant_gradient_keeps_the_step():
    """For a constant g, m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2 exactly, so
    every bias-corrected step is lr * g / (|g| + eps)."""
    g = np.array([1e-3, -0.5, 2.0, -7.0], np.float32)
    p = np.zeros(4, np.float32)
    out = run_oracle(p, [g] * 8, dict(HP, weight_decay=0.0))
    prev = p.astype(np.float64)
    for t, (pt, mt, vt) in enumerate(out, start=1):
        np.testing.assert_allclose(mt, (1 - 0.9 ** t) * g.astype(np.float64), rtol=1e-5)
        np.testing.assert_allclose(vt, (1 - 0.999 ** t) * g.astype(np.float64) ** 2, rtol=1e-4)
        np.testing.assert_allclose(pt - prev, -1e-3 * np.sign(g), rtol=1e-4)
        prev = pt.astype(np.float64)


def test_zero_gradient_only_decays():
    p = np.array([1.0, -3.0, 0.25, 1e-30], np.float32)
    (p1, m1, v1), = run_oracle(p, [np.zeros(4, np.float32)], dict(HP, weight_decay=0.1))
    decay = np.float32(1.0 - float(np.float32(1e-3)) * float(np.float32(0.1)))
    assert np.array_equal(p1, (decay * p).astype(np.float32))
    assert not np.any(m1) and not np.any(v1)


def test_each_rounding_exact_rationals():
    """One element through the fixed fp32 order, every operation redone on exact
    rationals and rounded once (sqrt checked by bracketing)."""
    rng = np.random.default_rng(4)
    for _ in range(40):
        p, g, m = (np.float32(x) for x in rng.standard_normal(3) * [0.1, 1e-2, 1e-3])
        v = np.float32(abs(rng.standard_normal()) * 1e-6)
        t = int(rng.integers(1, 50))
        sc = oracle.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t)
        p2, m2, v2 = oracle.adamw_update(np.array([p]), np.array([g]), np.array([m]),
                                         np.array([v]), sc)
        F = lambda x: Fraction(float(x))          # noqa: E731
        r = round_to_f32
        em = r(F(r(F(sc["b1"]) * F(m))) + F(r(F(sc["omb1"]) * F(g))))
        ev = r(F(r(F(sc["b2"]) * F(v))) + F(r(F(r(F(sc["omb2"]) * F(g))) * F(g))))
        assert m2[0] == np.float32(em) and v2[0] == np.float32(ev)
        s = float(np.sqrt(np.float32(ev)))
        ulp = float(np.spacing(np.float32(s)))
        assert (F(s) - F(ulp) / 2) ** 2 <= F(ev) <= (F(s) + F(ulp) / 2) ** 2
        den = r(F(r(F(s) * F(sc["inv_bc2"]))) + F(sc["eps"]))
        q = r(F(em) / F(den))
        ep = r(F(r(F(sc["decay"]) * F(p))) - F(r(F(sc["step_size"]) * F(q))))
        assert p2[0] == np.float32(ep)


ADAMW_HP = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (2e-4, 0.9, 0.95, 1e-6, 0.05),
            (3e-4, 0.8, 0.95, 1e-6, 0.1)]
STEPS = list(range(1, 41)) + [64, 100, 333, 1000, 4096, 10000]


def _neighbours(c):
    c = np.float32(c)
    return (Fraction(float(np.nextafter(c, np.float32(-np.inf)))), Fraction(float(c)),
            Fraction(float(np.nextafter(c, np.float32(np.inf)))))


@pytest.mark.parametrize("hp", ADAMW_HP)
def test_scalars_exact_definition(hp):
    """Every step scalar against its definition on exact rationals, with
    beta**t formed as an exact rational power: step_size and decay rounded by
    tests/exact.round_to_f32; inv_bc2 = 1/sqrt(1 - beta2**t) checked by
    bracketing it between the midpoints to its float32 neighbours (exact
    squares, no square root taken)."""
    lr, b1, b2, eps, wd = (Fraction(float(np.float32(v))) for v in hp)
    for t in STEPS:
        sc = oracle.adamw_scalars(*hp, t)
        assert float(sc["step_size"]) == round_to_f32(lr / (1 - b1 ** t)), t
        assert float(sc["decay"]) == round_to_f32(1 - lr * wd)
        assert float(sc["omb1"]) == round_to_f32(1 - b1)
        assert float(sc["omb2"]) == round_to_f32(1 - b2)
        q = 1 - b2 ** t
        lo, c, hi = _neighbours(sc["inv_bc2"])
        # 1/sqrt(q) lies between the midpoints (lo+c)/2 and (c+hi)/2
        assert ((lo + c) / 2) ** 2 * q <= 1 <= ((c + hi) / 2) ** 2 * q, t


def test_scalars_limits():
    """Closed forms: at t = 1 the bias-corrected step is lr/(1 - beta1) and
    inv_bc2 = 1/sqrt(1 - beta2); the step size falls monotonically towards lr
    and inv_bc2 towards 1; once beta**t is far below float32 resolution both
    are exactly lr and 1."""
    sc1 = oracle.adamw_scalars(1e-3, 0.5, 0.75, 1e-8, 0.0, 1)
    assert sc1["step_size"] == np.float32(2e-3)        # 0.5 is exact: lr / 0.5
    assert sc1["inv_bc2"] == np.float32(2.0)           # 1/sqrt(0.25)
    prev = None
    for t in (1, 2, 3, 5, 10, 30, 100, 300, 1000):
        sc = oracle.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, t)
        if prev is not None:
            assert sc["step_size"] <= prev["step_size"] and sc["inv_bc2"] <= prev["inv_bc2"]
        prev = sc
    far = oracle.adamw_scalars(1e-3, 0.9, 0.99, 1e-8, 0.0, 20000)
    assert far["step_size"] == np.float32(1e-3) and far["inv_bc2"] == np.float32(1.0)


def test_scalars_single_rounding_not_float64():
    """The scalars are the exact values rounded once, not a float64 value
    rounded again to float32: with the float32 lr = 11854442 * 2**-36 and
    wd = 11872131 * 2**-36, lr*wd = 2**-25 * (1 + 574 * 2**-47) (the integer
    product is 2**47 + 574).  1 - lr*wd then lies just below 1 - 2**-25, the
    midpoint between the float32 values 1 - 2**-24 and 1: float64 rounds it
    onto the midpoint and float32 then ties it to 1, while the exact value
    rounds down to 1 - 2**-24."""
    lr, wd = 11854442 * 2.0 ** -36, 11872131 * 2.0 ** -36
    assert np.float32(lr) == lr and np.float32(wd) == wd
    assert 11854442 * 11872131 == 2 ** 47 + 574
    exact = 1 - Fraction(lr) * Fraction(wd)
    assert 1 - Fraction(1, 2 ** 24) < exact < 1 - Fraction(1, 2 ** 25)
    assert np.float32(1.0 - lr * wd) == np.float32(1.0)     # float64 then float32
    sc = oracle.adamw_scalars(lr, 0.9, 0.999, 1e-8, wd, 1)
    assert float(sc["decay"]) == 1.0 - 2.0 ** -24 == round_to_f32(exact)


def test_frozen_a_keeps_a_and_its_moments():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((3, 16)).astype(np.float32)
    B = rng.standard_normal((8, 3)).astype(np.float32)
    dB = rng.standard_normal((8, 3)).astype(np.float32)
    mA = rng.standard_normal((3, 16)).astype(np.float32)
    z = np.zeros_like(B)
    A2, B2, mA2, vA2, mB2, vB2 = oracle.adapter_step_adamw(A, B, None, dB, mA, None, z, z,
                                                           1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    assert np.array_equal(A2, A) and np.array_equal(mA2, mA) and vA2 is None
    assert not np.array_equal(B2, B)


@pytest.mark.parametrize("mistake", ["no_bias_correction_1", "no_bias_correction_2",
                                     "no_decay", "eps_inside_sqrt"])
def test_planted_mistakes_are_caught(mistake, monkeypatch):
    """Each plausible slip, planted in the oracle, moves the first steps far
    outside the tolerance of the torch comparison above."""
    real_scalars, real_update = oracle.adamw_scalars, oracle.adamw_update

    def scalars(lr, b1, b2, eps, wd, t):
        sc = dict(real_scalars(lr, b1, b2, eps, wd, t))
        if mistake == "no_bias_correction_1":
            sc["step_size"] = np.float32(lr)
        elif mistake == "no_bias_correction_2":
            sc["inv_bc2"] = np.float32(1.0)
        elif mistake == "no_decay":
            sc["decay"] = np.float32(1.0)
        return sc

    def update(p, g, m, v, sc):
        if mistake != "eps_inside_sqrt":
            return real_update(p, g, m, v, sc)
        f = np.float32
        m2 = (sc["b1"] * m + sc["omb1"] * g).astype(f)
        v2 = (sc["b2"] * v + sc["omb2"] * g * g).astype(f)
        den = np.sqrt(v2 * sc["inv_bc2"] ** 2 + sc["eps"]).astype(f)
        return (sc["decay"] * p - sc["step_size"] * (m2 / den)).astype(f), m2, v2

    monkeypatch.setattr(oracle, "adamw_scalars", scalars)
    monkeypatch.setattr(oracle, "adamw_update", update)
    hp = dict(HP, weight_decay=0.1)
    p0, grads = problem(6, steps=2)
    ours = run_oracle(p0, grads, hp)
    ref = run_torch(p0, grads, hp)
    step = ours[0][0].astype(np.float64) - p0
    want = ref[0][0] - p0
    assert np.max(np.abs(step - want) / (np.abs(want) + 1e-12)) > 1e-3
