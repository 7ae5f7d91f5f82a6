"""melded_linear_fwd / melded_linear_bwd / adapter_step on the GPU against the
oracle: rel-L2 <= 1e-3 for Y, dX, dA, dB (fp32 accumulation); SGD bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3
from tests.gpu_util import (TOL, announce, check_elementwise, dev, gemm_bound, host, nan_f32,
                            rel_l2, rel_l2_rank, scalar)
import workloads as wl

pytestmark = pytest.mark.gpu


def quantized_problem(seed, T, d_in, d_out, r, x_std=1.0, dy_std=1e-2, b_std=1e-3):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    X = (rng.standard_normal((T, d_in)) * x_std).astype(np.float32)
    dY = (rng.standard_normal((T, d_out)) * dy_std).astype(np.float32)
    A = (rng.standard_normal((r, d_in)) / np.sqrt(max(r, 1))).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * b_std).astype(np.float32)
    wq, s_w, _, _ = oracle.fp8_quantize(W)
    xq, s_x, _, _ = oracle.fp8_quantize(X)
    gq, s_g, _, _ = oracle.fp8_quantize(dY)
    return dict(wq=wq, s_w=s_w, xq=xq, s_x=s_x, gq=gq, s_g=s_g, A=A, B=B)


def gpu_fwd(fq, p):
    T, d_out = p["xq"].shape[0], p["wq"].shape[0]
    y = nan_f32((T, d_out))
    fq.melded_linear_fwd(dev(p["xq"]), scalar(p["s_x"]), dev(p["wq"]), scalar(p["s_w"]), y)
    return host(y)


def gpu_bwd(fq, p, want_dx=True, want_da=True):
    T, d_out = p["gq"].shape
    d_in = p["xq"].shape[1]
    r = p["A"].shape[0]
    dx = torch.full((T, d_in), np.nan, dtype=torch.float32, device="cuda") if want_dx else None
    dA = torch.full((r, d_in), np.nan, dtype=torch.float32, device="cuda") if want_da else None
    dB = torch.full((d_out, r), np.nan, dtype=torch.float32, device="cuda")
    fq.melded_linear_bwd(dev(p["gq"]), scalar(p["s_g"]), dev(p["xq"]), scalar(p["s_x"]),
                         dev(p["wq"]), scalar(p["s_w"]), dev(p["A"]), dev(p["B"]), dx, dA, dB)
    return (host(dx) if want_dx else None), (host(dA) if want_da else None), host(dB)


SHAPES = [  # (T, d_in, d_out, r): full tiles, ragged tails in every dimension, tiny
    (256, 512, 512, 16),
    (257, 400, 272, 5),
    (600, 1040, 784, 64),
    (1, 16, 16, 1),
    (3, 48, 32, 70),
    (1000, 256, 1536, 128),
    (300, 384, 640, 8),      # K % 128 == 0 in both products: fast path with ragged M and N
    (513, 1152, 1280, 64),
    # ranks large enough that the backward contracts through G^^T X^ first
    (1024, 512, 512, 256),
    (512, 256, 384, 512),
]


@pytest.mark.parametrize("T,d_in,d_out,r", SHAPES)
def test_forward_parity(gpu_lib, T, d_in, d_out, r):
    announce(f"fwd T={T} d_in={d_in} d_out={d_out}")
    p = quantized_problem(T + d_in, T, d_in, d_out, r)
    y = gpu_fwd(gpu_lib, p)
    ref = oracle.melded_linear_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"])
    err = rel_l2(y, ref)
    bound = gemm_bound(e4m3.decode(p["xq"]), e4m3.decode(p["wq"]),
                       np.float64(p["s_x"]) * np.float64(p["s_w"]), ref)
    worst = check_elementwise(y, ref, bound, "Y")
    print(f"fwd rel-L2 {err:.3e}, worst error / per-element bound {worst:.3f}")
    assert err <= TOL


@pytest.mark.parametrize("T,d_in,d_out,r", SHAPES)
def test_backward_parity(gpu_lib, T, d_in, d_out, r):
    announce(f"bwd T={T} d_in={d_in} d_out={d_out} r={r}")
    p = quantized_problem(T + d_out, T, d_in, d_out, r)
    dx, dA, dB = gpu_bwd(gpu_lib, p)
    rdx, rdA, rdB = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"],
                                             p["s_w"], p["A"], p["B"])
    e = (rel_l2(dx, rdx), rel_l2(dA, rdA), rel_l2(dB, rdB))
    ek = (rel_l2_rank(dA, rdA, 0), rel_l2_rank(dB, rdB, 1))
    bound = gemm_bound(e4m3.decode(p["gq"]), e4m3.decode(p["wq"]).T,
                       np.float64(p["s_g"]) * np.float64(p["s_w"]), rdx)
    worst = check_elementwise(dx, rdx, bound, "dX")
    print("bwd rel-L2 dX %.3e dA %.3e dB %.3e; per rank component dA %.3e dB %.3e; "
          "dX worst / bound %.3f" % (e + ek + (worst,)))
    assert max(e) <= TOL and max(ek) <= TOL


def test_backward_frozen_a_and_no_dx(gpu_lib):
    announce("bwd frozen A, no dX")
    p = quantized_problem(3, 300, 512, 384, 32)
    _, _, dB = gpu_bwd(gpu_lib, p, want_dx=False, want_da=False)
    _, _, rdB = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"], p["s_w"],
                                         p["A"], p["B"], want_dx=False, want_da=False)
    assert rel_l2(dB, rdB) <= TOL


def test_backward_degenerate(gpu_lib):
    announce("bwd degenerate: T=0, B=0, r=0")
    p = quantized_problem(4, 0, 64, 48, 8)
    dx, dA, dB = gpu_bwd(gpu_lib, p)
    assert dx.shape == (0, 64) and not dA.any() and not dB.any()
    p = quantized_problem(5, 100, 64, 48, 8, b_std=0.0)
    _, dA, dB = gpu_bwd(gpu_lib, p)
    assert not dA.any()            # B = 0 => dA = 0 exactly
    p = quantized_problem(6, 100, 64, 48, 0)
    dx, dA, dB = gpu_bwd(gpu_lib, p)
    rdx, _, _ = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"], p["s_w"],
                                         p["A"], p["B"])
    assert dA.size == 0 and dB.size == 0 and rel_l2(dx, rdx) <= TOL


def test_full_size_attention_projection(gpu_lib):
    """4096 x 4096 weight, 4096 tokens with outlier channels, r = 64 (the 7B
    attention projection workload): every element of Y and dX against the
    oracle (rel-L2 and the per-element bound), dA and dB per rank
    component."""
    spec = wl.WORKLOADS[2].linears[0]
    announce("full-size 4096^3 fwd/bwd, every row")
    d = wl.make_linear(2, 0, spec, step=0)
    wq, s_w, _, _ = oracle.fp8_quantize(d["W"])
    xq, s_x, _, _ = oracle.fp8_quantize(d["X"])
    gq, s_g, _, _ = oracle.fp8_quantize(d["dY"])
    p = dict(wq=wq, s_w=s_w, xq=xq, s_x=s_x, gq=gq, s_g=s_g, A=d["A"], B=d["B"])
    y = gpu_fwd(gpu_lib, p)
    dx, dA, dB = gpu_bwd(gpu_lib, p)
    ry = oracle.melded_linear_fwd(xq, s_x, wq, s_w)
    rdx, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, d["A"], d["B"])
    xd, wd, gd = e4m3.decode(xq), e4m3.decode(wq), e4m3.decode(gq)
    wy = check_elementwise(y, ry, gemm_bound(xd, wd,
        np.float64(s_x) * np.float64(s_w), ry), "Y")
    wx = check_elementwise(dx, rdx, gemm_bound(gd, wd.T,
        np.float64(s_g) * np.float64(s_w), rdx), "dX")
    e = (rel_l2(y, ry), rel_l2(dx, rdx), rel_l2(dA, rdA), rel_l2(dB, rdB),
         rel_l2_rank(dA, rdA, 0), rel_l2_rank(dB, rdB, 1))
    print("full-size rel-L2 Y %.3e dX %.3e dA %.3e dB %.3e; per rank dA %.3e dB %.3e" % e
          + f"; worst / bound Y {wy:.3f} dX {wx:.3f}")
    assert max(e) <= TOL


def test_max_size_mlp_down(gpu_lib):
    """The largest single GEMM of the workloads: 7B MLP down projection,
    W 4096 x 11008, 8192 tokens.  Sampled rows of Y and dX."""
    announce("max-size fwd/bwd 8192 x 11008 -> 4096, sampled rows")
    rng = np.random.default_rng(77)
    T, d_in, d_out = 8192, 11008, 4096
    wq = rng.integers(0, 0x7F, size=(d_out, d_in), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(d_out, d_in), dtype=np.uint8) << 7)
    xq = rng.integers(0, 0x7F, size=(T, d_in), dtype=np.uint8)
    gq = rng.integers(0, 0x7F, size=(T, d_out), dtype=np.uint8)
    p = dict(wq=wq, s_w=np.float32(2000.0), xq=xq, s_x=np.float32(30.0), gq=gq,
             s_g=np.float32(5e4), A=np.zeros((1, d_in), np.float32), B=np.zeros((d_out, 1), np.float32))
    y = gpu_fwd(gpu_lib, p)
    dx, _, _ = gpu_bwd(gpu_lib, p, want_da=False)
    rows = np.array([0, 1, 4095, 4096, 5000, 8191])
    ry = oracle.melded_linear_fwd(xq[rows], p["s_x"], wq, p["s_w"])
    rdx, _, _ = oracle.melded_linear_bwd(gq[rows], p["s_g"], xq[rows], p["s_x"], wq, p["s_w"],
                                         p["A"], p["B"], want_da=False)
    assert rel_l2(y[rows], ry) <= TOL and rel_l2(dx[rows], rdx) <= TOL
    wd = e4m3.decode(wq)
    check_elementwise(y[rows], ry, gemm_bound(e4m3.decode(xq[rows]), wd,
        np.float64(p["s_x"]) * np.float64(p["s_w"]), ry), "Y")
    check_elementwise(dx[rows], rdx, gemm_bound(e4m3.decode(gq[rows]), wd.T,
        np.float64(p["s_g"]) * np.float64(p["s_w"]), rdx), "dX")


def test_adapter_step_bit_exact(gpu_lib):
    announce("adapter_step")
    rng = np.random.default_rng(11)
    for r, d_in, d_out in [(16, 512, 512), (5, 48, 80), (64, 4096, 4096)]:
        A = rng.standard_normal((r, d_in)).astype(np.float32)
        B = rng.standard_normal((d_out, r)).astype(np.float32)
        dA = rng.standard_normal((r, d_in)).astype(np.float32)
        dB = rng.standard_normal((d_out, r)).astype(np.float32)
        tA, tB = dev(A), dev(B)
        gpu_lib.adapter_step(tA, tB, dev(dA), dev(dB), 1e-3)
        rA, rB = oracle.adapter_step(A, B, dA, dB, 1e-3)
        assert np.array_equal(host(tA).view(np.uint32), rA.view(np.uint32))
        assert np.array_equal(host(tB).view(np.uint32), rB.view(np.uint32))
        tA2 = dev(A)
        gpu_lib.adapter_step(tA2, dev(B), None, dev(dB), 1e-3)     # frozen A
        assert np.array_equal(host(tA2), A)


def test_backward_is_deterministic(gpu_lib):
    announce("bwd twice, bitwise equal")
    p = quantized_problem(12, 777, 512, 640, 64)
    a = gpu_bwd(gpu_lib, p)
    b = gpu_bwd(gpu_lib, p)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_split_last_round_parity_and_determinism(gpu_lib):
    """A tile count just past the CU count (16 x 17 = 272 tiles of 256 x 256
    on 256 CUs) with a long K (8192 = 64 steps): the 16 tiles of the last
    round run as two K halves added into a zeroed output.  Y in full against
    the oracle, bitwise equal over two runs.  Then a dX product whose four
    tiles are all split, with an odd number of K steps (8320 = 65: halves of
    32 and 33).  Outputs are NaN-filled beforehand, so an element left
    unwritten shows."""
    announce("fwd 4096 x 8192 -> 4352 (split last round), full Y")
    p = quantized_problem(21, 4096, 8192, 4352, 1)
    T, d_out = 4096, 4352

    def fwd():
        y = torch.full((T, d_out), np.nan, dtype=torch.float32, device="cuda")
        gpu_lib.melded_linear_fwd(dev(p["xq"]), scalar(p["s_x"]), dev(p["wq"]),
                                  scalar(p["s_w"]), y)
        return host(y)
    y1, y2 = fwd(), fwd()
    ry = oracle.melded_linear_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"])
    assert np.isfinite(y1).all() and rel_l2(y1, ry) <= TOL
    check_elementwise(y1, ry, gemm_bound(e4m3.decode(p["xq"]), e4m3.decode(p["wq"]),
        np.float64(p["s_x"]) * np.float64(p["s_w"]), ry), "Y")
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    del p
    announce("bwd 256 x 8320 -> 1024 (every dX tile split, odd K steps)")
    q = quantized_problem(22, 256, 1024, 8320, 3)
    dx1, _, dB1 = gpu_bwd(gpu_lib, q, want_da=False)
    dx2, _, _ = gpu_bwd(gpu_lib, q, want_da=False)
    rdx, _, rdB = oracle.melded_linear_bwd(q["gq"], q["s_g"], q["xq"], q["s_x"], q["wq"],
                                           q["s_w"], q["A"], q["B"], want_da=False)
    assert np.isfinite(dx1).all() and rel_l2(dx1, rdx) <= TOL and rel_l2(dB1, rdB) <= TOL
    check_elementwise(dx1, rdx, gemm_bound(e4m3.decode(q["gq"]), e4m3.decode(q["wq"]).T,
        np.float64(q["s_g"]) * np.float64(q["s_w"]), rdx), "dX")
    assert np.array_equal(dx1.view(np.uint32), dx2.view(np.uint32))


def test_fp8_matrix_core_block_truncation(gpu_lib):
    """The accumulation model the per-element bound (tests/gpu_util.py,
    gemm_bound) rests on, observed through melded_linear_fwd with unit scales
    (K = 128 and K = 64 + 16, i.e. both GEMM kernels): products of an
    aligned block of 8 consecutive K positions are aligned to the block's
    largest exponent sum E and truncated toward zero to multiples of
    2^(E-13); products in other blocks are not.  Here the block's large
    product is 128 * 128 = 2^14, so a small product p in the same block
    contributes trunc(p / 2) * 2, one in the next block contributes p."""
    announce("FP8 matrix-core block truncation, through melded_linear_fwd")
    code = {v: int(e4m3.encode(np.array([v], np.float32))[0]) for v in
            (128.0, 1.0, 7.0, -7.0, 1.875, 15.0, 0.75)}
    smalls = [7.0, -7.0, 1.875, 15.0, 0.75]
    for K in (128, 80):
        rows = []
        for pos in (1, 8):                       # same block as k = 0, next block
            for v in smalls:
                x = np.zeros(K, np.uint8)
                x[0], x[pos] = code[128.0], code[v]
                rows.append((x, v, pos))
        xq = np.stack([r[0] for r in rows])
        wq = np.zeros((16, K), np.uint8)
        wq[0, 0], wq[0, 1], wq[0, 8] = code[128.0], code[1.0], code[1.0]
        y = gpu_fwd(gpu_lib, dict(xq=xq, s_x=np.float32(1.0), wq=wq, s_w=np.float32(1.0)))
        for i, (_, v, pos) in enumerate(rows):
            want = 16384.0 + (np.trunc(v / 2.0) * 2.0 if pos == 1 else v)
            assert y[i, 0] == np.float32(want), (K, pos, v, y[i, 0], want)


def test_backward_wide_route_e5m2(gpu_lib):
    """A large-rank backward (through G^^T X^) with an E5M2 upstream gradient
    (the FP8 product G~^T X~ then takes the E5M2 operand)."""
    announce("bwd large rank, E5M2 gradient")
    rng = np.random.default_rng(41)
    T, d_in, d_out, r = 1024, 512, 384, 320
    p = quantized_problem(41, T, d_in, d_out, r)
    dY = (rng.standard_normal((T, d_out)) * 1e-2).astype(np.float32)
    gq, s_g, _, _ = oracle.fp8_quantize(dY, fmt="e5m2")
    dx = torch.full((T, d_in), np.nan, dtype=torch.float32, device="cuda")
    dA = torch.full((r, d_in), np.nan, dtype=torch.float32, device="cuda")
    dB = torch.full((d_out, r), np.nan, dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_bwd(dev(gq), scalar(s_g), dev(p["xq"]), scalar(p["s_x"]), dev(p["wq"]),
                              scalar(p["s_w"]), dev(p["A"]), dev(p["B"]), dx, dA, dB,
                              g_fmt="e5m2")
    rdx, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, p["xq"], p["s_x"], p["wq"], p["s_w"],
                                             p["A"], p["B"], g_fmt="e5m2")
    e = (rel_l2(host(dx), rdx), rel_l2(host(dA), rdA), rel_l2(host(dB), rdB),
         rel_l2_rank(host(dA), rdA, 0), rel_l2_rank(host(dB), rdB, 1))
    print("wide E5M2 bwd rel-L2 dX %.2e dA %.2e dB %.2e per rank %.2e %.2e" % e)
    assert max(e) <= TOL
