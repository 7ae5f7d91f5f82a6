"""Pins of the oracle's two comparison layers (oracle/baselines.py): the
separate-path FP8 LoRA layer and the bfloat16 LoRA layer.

* bfloat16 rounding against torch's own conversion (an independent library
  routine) and hand-derived ties;
* both layers against the melded layer's exact formulas on inputs where every
  quantization and every bfloat16 rounding is exact (values on the formats'
  grids with power-of-two scales): then the three layers must agree to the
  last bit of float32, which fixes which operand meets which in every
  product, every transpose and every scale;
* closed forms: B = 0 leaves the backbone product alone and gives dA = 0;
* the separate path differs from the melded layer by quantization noise of
  the size the E4M3 grid allows, no more.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import baselines as bl
from oracle import e4m3


def test_bf16_round_against_torch_and_ties():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.uniform(-30, 30, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40], np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bl.bf16_round(x).view(np.uint32), ref.view(np.uint32))
    # hand-derived: 1 + 2^-8 is half-way between 1 and 1 + 2^-7 -> 1 (even);
    # 1 + 3 * 2^-8 is half-way between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6 (even)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20],
                    np.float32)
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7], np.float32)
    assert np.array_equal(bl.bf16_round(ties), want)


def code_of(v):
    return int(e4m3.encode(np.array([v], np.float32))[0])


def exact_problem(seed, T=32, d_in=48, d_out=32, r=8, lim=7):
    """X^, W^, G^ on {0, +-1} with unit scales, A and B on {0, +-c} with the
    extremes present (so Q(A), Q(B) are exact), and U = X^ A^T, V = G^ B
    integer multiples of c with |count| <= lim and the maximum lim reached:
    then Q(U), Q(V) are exact too (lim * c maps to 448; lim <= 7 keeps every
    multiple on the E4M3 grid) and so is every bfloat16 rounding."""
    rng = np.random.default_rng(seed)
    for _ in range(20000):
        xs = rng.choice([-1, 0, 0, 0, 1], size=(T, d_in))
        gs = rng.choice([-1, 0, 0, 0, 1], size=(T, d_out))
        a = rng.choice([-1, 0, 0, 0, 0, 0, 1], size=(r, d_in))
        b = rng.choice([-1, 0, 0, 0, 0, 0, 1], size=(d_out, r))
        u = xs @ a.T
        v = gs @ b
        if (np.abs(u).max() == lim and np.abs(v).max() == lim and np.abs(a).max() == 1
                and np.abs(b).max() == 1):
            break
    else:
        raise RuntimeError("no exact problem found")
    c_a, c_b = 2.0 ** -3, 2.0 ** -2
    code = {1: code_of(1.0), -1: code_of(-1.0), 0: 0}
    enc = np.vectorize(lambda t: code[int(t)])
    xq = enc(xs).astype(np.uint8)
    gq = enc(gs).astype(np.uint8)
    wq = rng.choice([code_of(v) for v in (-2.0, -1.0, 0.5, 1.0, 3.0)], size=(d_out, d_in)).astype(np.uint8)
    one = np.float32(1.0)
    return dict(xs=xs.astype(np.float64), gs=gs.astype(np.float64), xq=xq, gq=gq, wq=wq,
                A=(a * c_a).astype(np.float32), B=(b * c_b).astype(np.float32), s=one)


def melded_exact(p):
    """The melded layer's formulas in float64 with X^ = X, G^ = G."""
    X, G, W = p["xs"], p["gs"], e4m3.decode(p["wq"])
    A, B = p["A"].astype(np.float64), p["B"].astype(np.float64)
    U, V = X @ A.T, G @ B
    return dict(y0=X @ W.T, ylora=U @ B.T, dx0=G @ W, dxlora=V @ A, dB=G.T @ U, dA=V.T @ X)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_separate_fp8_equals_exact_formulas_on_exact_inputs(seed):
    p = exact_problem(seed)
    m = melded_exact(p)
    s = p["s"]
    y, sv = bl.lora_separate_fp8_fwd(p["xq"], s, p["wq"], s, p["A"], p["B"])
    # every quantization on the way is exact
    assert np.array_equal(e4m3.decode(sv["aq"]) / np.float64(sv["s_a"]), p["A"])
    assert np.array_equal(e4m3.decode(sv["uq"]) / np.float64(sv["s_u"]),
                          p["xs"] @ p["A"].astype(np.float64).T)
    assert np.array_equal(y, (m["y0"] + m["ylora"]).astype(np.float32))
    dx, dA, dB, vq, s_v, _ = bl.lora_separate_fp8_bwd(p["gq"], s, p["xq"], s, p["wq"], s, sv)
    assert np.array_equal(dx, (m["dx0"] + m["dxlora"]).astype(np.float32))
    assert np.array_equal(dB, m["dB"].astype(np.float32))
    assert np.array_equal(dA, m["dA"].astype(np.float32))
    # and these are the melded oracle's adapter gradients
    _, mdA, mdB = oracle.melded_linear_bwd(p["gq"], s, p["xq"], s, p["wq"], s, p["A"], p["B"])
    assert np.array_equal(dA, mdA) and np.array_equal(dB, mdB)


@pytest.mark.parametrize("seed", [4, 5])
def test_bf16_equals_exact_formulas_on_exact_inputs(seed):
    p = exact_problem(seed)
    m = melded_exact(p)
    s = p["s"]
    X = p["xs"].astype(np.float32)
    dY = p["gs"].astype(np.float32)
    y, ub = bl.lora_bf16_fwd(X, p["xq"], s, p["wq"], s, p["A"], p["B"])
    assert np.array_equal(y, (m["y0"] + m["ylora"]).astype(np.float32))
    dx, dA, dB, _ = bl.lora_bf16_bwd(dY, p["gq"], s, X, p["wq"], s, p["A"], p["B"], ub)
    assert np.array_equal(dx, (m["dx0"] + m["dxlora"]).astype(np.float32))
    assert np.array_equal(dB, m["dB"].astype(np.float32))
    assert np.array_equal(dA, m["dA"].astype(np.float32))


def random_problem(seed, T=64, d_in=96, d_out=80, r=16, b_std=0.5):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    dY = (rng.standard_normal((T, d_out)) * 1e-2).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((r, d_in)) / np.sqrt(r)).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * b_std).astype(np.float32)
    xq, s_x, _, _ = oracle.fp8_quantize(X)
    gq, s_g, _, _ = oracle.fp8_quantize(dY)
    wq, s_w, _, _ = oracle.fp8_quantize(W)
    return dict(X=X, dY=dY, A=A, B=B, xq=xq, s_x=s_x, gq=gq, s_g=s_g, wq=wq, s_w=s_w)


def test_zero_B_leaves_the_backbone():
    p = random_problem(7, b_std=0.0)
    y, sv = bl.lora_separate_fp8_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"], p["A"], p["B"])
    assert np.array_equal(y, oracle.melded_linear_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"]))
    dx, dA, dB, _, _, _ = bl.lora_separate_fp8_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"],
                                                   p["s_w"], sv)
    rdx, _, _ = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"], p["s_w"],
                                         p["A"], p["B"])
    assert not dA.any() and np.array_equal(dx, rdx)
    yb, ub = bl.lora_bf16_fwd(p["X"], p["xq"], p["s_x"], p["wq"], p["s_w"], p["A"], p["B"])
    assert np.array_equal(yb, y)
    _, dAb, _, _ = bl.lora_bf16_bwd(p["dY"], p["gq"], p["s_g"], p["X"], p["wq"], p["s_w"], p["A"],
                                    p["B"], ub)
    assert not dAb.any()


def test_separate_path_within_quantization_noise_of_melded():
    """The separate path's adapter gradients differ from the melded layer's
    (which keep X A^T and G B unquantized) by E4M3 rounding of U, V, A and B:
    a few per cent, and no more than the E4M3 half-step (2^-4 relative)
    bounds."""
    p = random_problem(8, T=256, d_in=128, d_out=96, r=16)
    _, sv = bl.lora_separate_fp8_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"], p["A"], p["B"])
    _, dA, dB, _, _, _ = bl.lora_separate_fp8_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"],
                                                  p["s_w"], sv)
    _, mdA, mdB = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"],
                                           p["s_w"], p["A"], p["B"])
    for g, ref in ((dA, mdA), (dB, mdB)):
        e = np.linalg.norm(g.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert 1e-3 < e < 2 * 2.0 ** -4, e
