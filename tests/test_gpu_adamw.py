"""adapter_step_adamw on the GPU against the oracle: weights and both moments
bit-exact over consecutive steps (every float operation of the update is
rounded on its own on both sides; sqrt and division are correctly rounded),
the step count advanced in the device-side state."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


def state_at(gpu_lib, t, beta1=None, beta2=None):
    """An AdamW state after t steps: the next call takes step t + 1 (the
    library derives every step scalar from the step count alone)."""
    st = gpu_lib.adamw_state()
    h = np.zeros(8, np.int64)
    h[0] = t
    st.copy_(torch.from_numpy(h))
    return st


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def grads(rng, shape):
    """gradients over many decades, with zeros and values whose squares are
    subnormal or underflow"""
    g = rng.standard_normal(shape) * 10.0 ** rng.uniform(-24, 1, shape)
    g[rng.random(shape) < 0.02] = 0.0
    return g.astype(np.float32)


@pytest.mark.parametrize("r,d_in,d_out", [(16, 512, 512), (3, 37, 13), (64, 4096, 4096),
                                          (1, 1, 5)])
def test_adamw_bit_exact_over_steps(gpu_lib, r, d_in, d_out):
    announce(f"adapter_step_adamw r {r} d_in {d_in} d_out {d_out}")
    rng = np.random.default_rng(r * 1000 + d_in)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    A = (rng.standard_normal((r, d_in)) / np.sqrt(r)).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * 1e-3).astype(np.float32)
    st = [A, B, np.zeros_like(A), np.zeros_like(A), np.zeros_like(B), np.zeros_like(B)]
    tA, tB, tmA, tvA, tmB, tvB = (dev(x) for x in st)
    state = gpu_lib.adamw_state()
    for step in (1, 2, 3, 1000):
        dA, dB = grads(rng, A.shape), grads(rng, B.shape)
        if step == 1000:                    # jump ahead: the state after 999 steps
            state = state_at(gpu_lib, 999, hp["beta1"], hp["beta2"])
        gpu_lib.adapter_step_adamw(tA, tB, dev(dA), dev(dB), tmA, tvA, tmB, tvB, state, **hp)
        assert int(host(state)[0]) == step
        A2, B2, mA2, vA2, mB2, vB2 = oracle.adapter_step_adamw(
            st[0], st[1], dA, dB, st[2], st[3], st[4], st[5], hp["lr"], hp["beta1"],
            hp["beta2"], hp["eps"], hp["weight_decay"], step)
        st = [A2, B2, mA2, vA2, mB2, vB2]
        for name, t, ref in zip(["A", "B", "mA", "vA", "mB", "vB"],
                                [tA, tB, tmA, tvA, tmB, tvB], st):
            got = host(t)
            assert np.array_equal(bits(got), bits(ref)), (step, name)


def test_adamw_frozen_a_and_hyper_parameters(gpu_lib):
    announce("adapter_step_adamw frozen A, beta2 0.95, wd 0.1")
    rng = np.random.default_rng(7)
    r, d_in, d_out = 8, 64, 96
    A = rng.standard_normal((r, d_in)).astype(np.float32)
    B = rng.standard_normal((d_out, r)).astype(np.float32)
    mB = (rng.standard_normal((d_out, r)) * 1e-3).astype(np.float32)
    vB = (rng.random((d_out, r)) * 1e-6).astype(np.float32)
    dB = grads(rng, B.shape)
    tA, tB, tmB, tvB = dev(A), dev(B), dev(mB), dev(vB)
    hp = dict(lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1)
    state = state_at(gpu_lib, 16, hp["beta1"], hp["beta2"])
    gpu_lib.adapter_step_adamw(tA, tB, None, dev(dB), None, None, tmB, tvB, state, **hp)
    _, B2, _, _, mB2, vB2 = oracle.adapter_step_adamw(A, B, None, dB, None, None, mB, vB,
                                                      hp["lr"], hp["beta1"], hp["beta2"],
                                                      hp["eps"], hp["weight_decay"], 17)
    assert np.array_equal(host(tA), A)
    for t, ref in ((tB, B2), (tmB, mB2), (tvB, vB2)):
        assert np.array_equal(bits(host(t)), bits(ref))


def test_adamw_empty(gpu_lib):
    announce("adapter_step_adamw r = 0")
    z = torch.zeros((0, 32), device="cuda")
    zb = torch.zeros((48, 0), device="cuda")
    state = gpu_lib.adamw_state()
    gpu_lib.adapter_step_adamw(z, zb, z, zb, z, z, zb, zb, state, lr=1e-3)
    assert int(host(state)[0]) == 1                 # the step is counted


@pytest.mark.parametrize("hp,steps", [
    (dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01), 10000),
    (dict(lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1), 2000),
    # lr * wd = 2^-25 (1 + 574 2^-47): 1 - lr*wd rounded through float64
    # would tie to 1.0; the exact value rounds to 1 - 2^-24
    (dict(lr=11854442 * 2.0 ** -36, beta1=0.5, beta2=0.75, eps=1e-8,
          weight_decay=11872131 * 2.0 ** -36), 200)])
def test_adamw_step_scalars_trace(gpu_lib, hp, steps):
    """The float32 step scalars the state holds after each of `steps`
    consecutive calls (tiny tensors), bit for bit against the oracle's
    exact-definition values: decay, 1 - beta, lr / (1 - beta1^t) and
    1 / sqrt(1 - beta2^t)."""
    announce(f"adapter_step_adamw scalar trace, {steps} steps, {hp}")
    z = torch.zeros((1, 16), device="cuda")
    zb = torch.zeros((16, 1), device="cuda")
    state = gpu_lib.adamw_state()
    hist = torch.empty((steps, 8), dtype=torch.int64, device="cuda")
    for i in range(steps):
        gpu_lib.adapter_step_adamw(z, zb, z, zb, z, z, zb, zb, state, **hp)
        hist[i].copy_(state)
    h = host(hist)
    assert np.array_equal(h[:, 0], np.arange(1, steps + 1))
    sc = h[:, 3:7].copy().view(np.float32)          # b1 b2 omb1 omb2 eps decay step inv
    names = ["b1", "b2", "omb1", "omb2", "eps", "decay", "step_size", "inv_bc2"]
    for i in range(steps):
        ref = oracle.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                   hp["weight_decay"], i + 1)
        got = dict(zip(names, sc[i]))
        for k in names:
            assert bits(got[k]) == bits(ref[k]), (i + 1, k, got[k], ref[k])
