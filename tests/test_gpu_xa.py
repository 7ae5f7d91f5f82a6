"""melded_linear_fwd_xa / melded_linear_bwd_xa on the GPU against the oracle.

The pair computes what melded_linear_fwd + melded_linear_bwd compute, with
the rank-r factor X^ A^T formed in the forward call (inside the FP8 product's
tiles where the shape allows) and handed to the backward call, which forms
G^ B inside the dX product.  Checked here: Y per element against the FP8
product bound, X^ A^T against its exact value (rel-L2, per rank column), and
dX, dA, dB against oracle.melded_linear_bwd (rel-L2 <= 1e-3, per rank
component for dA and dB), on shapes that take the fused route and on shapes
that fall back to the separate kernels."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3
from tests.gpu_util import (TOL, announce, check_elementwise, dev, gemm_bound, host, nan_f32,
                            rel_l2, rel_l2_rank, scalar)
from tests.test_gpu_linear import quantized_problem
import workloads as wl

pytestmark = pytest.mark.gpu


def gpu_pair(fq, p, g_fmt="e4m3", gq=None, s_g=None):
    gq = p["gq"] if gq is None else gq
    s_g = p["s_g"] if s_g is None else s_g
    T, d_in = p["xq"].shape
    d_out = p["wq"].shape[0]
    r = p["A"].shape[0]
    xq, wq, A, B = dev(p["xq"]), dev(p["wq"]), dev(p["A"]), dev(p["B"])
    sx, sw = scalar(p["s_x"]), scalar(p["s_w"])
    y, xa = nan_f32((T, d_out)), nan_f32((T, r))
    fq.melded_linear_fwd_xa(xq, sx, wq, sw, A, y, xa)
    dx, dA, dB = nan_f32((T, d_in)), nan_f32((r, d_in)), nan_f32((d_out, r))
    fq.melded_linear_bwd_xa(dev(gq), scalar(s_g), xq, sx, wq, sw, A, B, xa, dx, dA, dB,
                            g_fmt=g_fmt)
    return host(y), host(xa), host(dx), host(dA), host(dB)


def exact_xa(p):
    return e4m3.decode(p["xq"]) @ np.asarray(p["A"], np.float64).T / np.float64(p["s_x"])


XA_SHAPES = [  # (T, d_in, d_out, r, fused)
    (512, 1024, 1024, 16, True),
    (600, 1024, 1280, 16, True),      # ragged T and a 5-tile N
    (1024, 2048, 2048, 32, True),
    (384, 2048, 1024, 13, True),      # rank not a multiple of the 16-row piece tile
    (9000, 1024, 1024, 8, True),      # two token splits of 36 steps: three 16-step windows of
                                      # scale bytes each (a buffer reused), a clamped last one
    (256, 512, 512, 16, False),       # too few column tiles to carry the pieces
    (257, 400, 272, 5, False),        # K not a multiple of 128
    (300, 384, 640, 8, False),
    (512, 512, 384, 100, False),      # two 64-rank tiles, the second ragged
]


@pytest.mark.parametrize("T,d_in,d_out,r,fused", XA_SHAPES)
def test_xa_pair_parity(gpu_lib, T, d_in, d_out, r, fused):
    announce(f"fwd_xa/bwd_xa T={T} d_in={d_in} d_out={d_out} r={r}")
    assert gpu_lib.melded_linear_xa_fused(T, d_in, d_out, r) == fused
    p = quantized_problem(T + 3 * r, T, d_in, d_out, r, b_std=0.5)
    y, xa, dx, dA, dB = gpu_pair(gpu_lib, p)
    ref_y = oracle.melded_linear_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"])
    worst_y = check_elementwise(
        y, ref_y, gemm_bound(e4m3.decode(p["xq"]), e4m3.decode(p["wq"]),
                             np.float64(p["s_x"]) * np.float64(p["s_w"]), ref_y), "Y")
    xa64 = exact_xa(p)
    e_xa = (rel_l2(xa, xa64), rel_l2_rank(xa, xa64, 1))
    rdx, rdA, rdB = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"],
                                             p["s_w"], p["A"], p["B"])
    worst_dx = check_elementwise(
        dx, rdx, gemm_bound(e4m3.decode(p["gq"]), e4m3.decode(p["wq"]).T,
                            np.float64(p["s_g"]) * np.float64(p["s_w"]), rdx), "dX")
    e = (rel_l2(dx, rdx), rel_l2(dA, rdA), rel_l2(dB, rdB), rel_l2_rank(dA, rdA, 0),
         rel_l2_rank(dB, rdB, 1))
    print("xa pair: X^A^T rel-L2 %.2e (per rank %.2e); dX %.2e dA %.2e dB %.2e (per rank %.2e "
          "%.2e); worst / bound Y %.3f dX %.3f" % (e_xa + e + (worst_y, worst_dx)))
    assert max(e_xa) <= TOL and max(e) <= TOL


def test_xa_pair_e5m2_gradient(gpu_lib):
    """The fused backward with an E5M2 upstream gradient (G~ the E5M2 operand
    of the dX product that also forms G^ B)."""
    T, d_in, d_out, r = 512, 1024, 1024, 16
    announce(f"fwd_xa/bwd_xa E5M2 gradient T={T} d={d_in} r={r}")
    assert gpu_lib.melded_linear_xa_fused(T, d_in, d_out, r)
    p = quantized_problem(77, T, d_in, d_out, r, b_std=0.5)
    dY = (np.random.default_rng(78).standard_normal((T, d_out)) * 1e-2).astype(np.float32)
    gq, s_g, _, _ = oracle.fp8_quantize(dY, fmt="e5m2")
    _, _, dx, dA, dB = gpu_pair(gpu_lib, p, g_fmt="e5m2", gq=gq, s_g=s_g)
    rdx, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, p["xq"], p["s_x"], p["wq"], p["s_w"],
                                             p["A"], p["B"], g_fmt="e5m2")
    e = (rel_l2(dx, rdx), rel_l2(dA, rdA), rel_l2(dB, rdB), rel_l2_rank(dA, rdA, 0),
         rel_l2_rank(dB, rdB, 1))
    print("xa pair E5M2: dX %.2e dA %.2e dB %.2e (per rank %.2e %.2e)" % e)
    assert max(e) <= TOL


def test_xa_pair_agrees_with_unfused_calls(gpu_lib):
    """Same inputs through melded_linear_fwd + melded_linear_bwd: Y is the
    same FP8 product (bit for bit), and the gradients agree to the two
    routes' rounding."""
    T, d_in, d_out, r = 512, 1024, 1024, 16
    announce(f"fwd_xa/bwd_xa against fwd/bwd T={T} d={d_in} r={r}")
    p = quantized_problem(91, T, d_in, d_out, r, b_std=0.5)
    y, _, dx, dA, dB = gpu_pair(gpu_lib, p)
    fq = gpu_lib
    y1 = nan_f32((T, d_out))
    fq.melded_linear_fwd(dev(p["xq"]), scalar(p["s_x"]), dev(p["wq"]), scalar(p["s_w"]), y1)
    dx1, dA1, dB1 = nan_f32((T, d_in)), nan_f32((r, d_in)), nan_f32((d_out, r))
    fq.melded_linear_bwd(dev(p["gq"]), scalar(p["s_g"]), dev(p["xq"]), scalar(p["s_x"]),
                         dev(p["wq"]), scalar(p["s_w"]), dev(p["A"]), dev(p["B"]), dx1, dA1, dB1)
    assert np.array_equal(y, host(y1))
    assert np.array_equal(dx, host(dx1))
    assert rel_l2(dA, host(dA1)) <= TOL and rel_l2(dB, host(dB1)) <= TOL


def test_xa_pair_degenerate(gpu_lib):
    announce("fwd_xa/bwd_xa degenerate: r=0, T=0, B=0")
    p = quantized_problem(5, 100, 64, 48, 0)
    y, xa, dx, dA, dB = gpu_pair(gpu_lib, p)
    ref_y = oracle.melded_linear_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"])
    rdx, _, _ = oracle.melded_linear_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"], p["s_w"],
                                         p["A"], p["B"])
    assert xa.size == dA.size == dB.size == 0
    assert rel_l2(y, ref_y) <= TOL and rel_l2(dx, rdx) <= TOL
    p = quantized_problem(6, 0, 1024, 1024, 16)
    y, xa, dx, dA, dB = gpu_pair(gpu_lib, p)
    assert y.size == 0 and not dA.any() and not dB.any()
    p = quantized_problem(7, 512, 1024, 1024, 16, b_std=0.0)
    _, _, _, dA, _ = gpu_pair(gpu_lib, p)
    assert not dA.any()            # B = 0 => G^ B = 0 => dA = 0 exactly


@pytest.mark.parametrize("cfg", [2, 4])
def test_xa_pair_full_size_attention_projection(gpu_lib, cfg):
    """The 7B attention projection (4096 x 4096 weight, 4096 tokens with
    outlier channels, r = 64) and the 13B q projection (5120 x 5120: 320
    output tiles, so the last four tile columns of the forward and dX
    products run as 128 x 128 tiles in a launch of their own) through the
    fused pair: sampled rows of Y and dX against the oracle row by row (each
    row depends on its own row of X~ or G~ only; every column is checked),
    X^ A^T and dA, dB complete."""
    spec = wl.WORKLOADS[cfg].linears[0]
    T, d_in, d_out, r = spec.tokens, spec.d_in, spec.d_out, spec.rank
    announce(f"fwd_xa/bwd_xa full size T={T} d_in={d_in} d_out={d_out} r={r}")
    assert gpu_lib.melded_linear_xa_fused(T, d_in, d_out, r)
    d = wl.make_linear(cfg, 0, spec, step=0)
    wq, s_w, _, _ = oracle.fp8_quantize(d["W"])
    xq, s_x, _, _ = oracle.fp8_quantize(d["X"])
    gq, s_g, _, _ = oracle.fp8_quantize(d["dY"])
    p = dict(wq=wq, s_w=s_w, xq=xq, s_x=s_x, gq=gq, s_g=s_g, A=d["A"], B=d["B"])
    y, xa, dx, dA, dB = gpu_pair(gpu_lib, p)
    rows = np.random.default_rng(12).choice(T, 96, replace=False)
    ref_y = oracle.melded_linear_fwd(xq[rows], s_x, wq, s_w)
    check_elementwise(y[rows], ref_y,
                      gemm_bound(e4m3.decode(xq[rows]), e4m3.decode(wq),
                                 np.float64(s_x) * np.float64(s_w), ref_y), "Y")
    rdx, _, _ = oracle.melded_linear_bwd(gq[rows], s_g, xq[rows], s_x, wq, s_w, p["A"], p["B"],
                                         want_da=False)
    check_elementwise(dx[rows], rdx,
                      gemm_bound(e4m3.decode(gq[rows]), e4m3.decode(wq).T,
                                 np.float64(s_g) * np.float64(s_w), rdx), "dX")
    xa64 = exact_xa(p)
    _, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, p["A"], p["B"],
                                           want_dx=False)
    e = (rel_l2(y[rows], ref_y), rel_l2(dx[rows], rdx), rel_l2(xa, xa64),
         rel_l2_rank(xa, xa64, 1), rel_l2(dA, rdA), rel_l2(dB, rdB), rel_l2_rank(dA, rdA, 0),
         rel_l2_rank(dB, rdB, 1))
    print("full-size xa pair: Y %.2e dX %.2e X^A^T %.2e (per rank %.2e) dA %.2e dB %.2e "
          "(per rank %.2e %.2e)" % e)
    assert max(e) <= TOL


@pytest.mark.parametrize("T,d_in,d_out,r", [(1024, 2048, 2048, 32), (2048, 4096, 4096, 64)])
def test_xa_pair_is_deterministic(gpu_lib, T, d_in, d_out, r):
    """The same inputs twice give the same bits: the first shape splits the
    token contraction into two halves added with float atomics onto zeroed
    outputs (two addends on a zero: order-independent), the second runs it
    as one split with plain stores."""
    announce(f"fwd_xa/bwd_xa determinism T={T} d={d_in} r={r}")
    p = quantized_problem(5 + r, T, d_in, d_out, r, b_std=0.5)
    first = gpu_pair(gpu_lib, p)
    second = gpu_pair(gpu_lib, p)
    for a, b in zip(first, second):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def pieces_regions(r, d_in):
    """Byte ranges of A's pieces buffer that hold data (pieces.hpp's layout:
    three planes of r rounded up to 16 rows of d_in codes, then, 256-byte
    aligned, d_in / 128 x rows x 4 scale bytes); the rest is padding."""
    rp = (r + 15) // 16 * 16
    planes = 3 * rp * d_in
    e0 = (planes + 255) // 256 * 256
    return [(0, planes), (e0, e0 + d_in // 128 * rp * 4)]


@pytest.mark.parametrize("T,d_in,d_out,r", [(384, 2048, 1024, 13), (1024, 2048, 2048, 32),
                                            (4096, 4096, 4096, 64), (64, 256, 301, 13)])
def test_adapter_pieces_path(gpu_lib, T, d_in, d_out, r):
    """A's pieces kept by the optimizer: adapter_step_pieces gives A and B bit
    for bit as adapter_step and the same pieces as adapter_pieces on the new
    A (every data byte written: the same result over two different
    prefills), and melded_linear_fwd_xa_pieces gives Y and xa bit for bit as
    melded_linear_fwd_xa from A.  The last shape has d_out * r not a multiple
    of 4 (B's tail) and too few column tiles for the fused forward."""
    fq = gpu_lib
    announce(f"adapter pieces T={T} d_in={d_in} d_out={d_out} r={r}")
    p = quantized_problem(211, T, d_in, d_out, r, b_std=0.5)
    rng = np.random.default_rng(212)
    gA = dev((rng.standard_normal((r, d_in)) * 1e-2).astype(np.float32))
    gB = dev((rng.standard_normal((d_out, r)) * 1e-2).astype(np.float32))
    lr = 0.37
    nb = fq.adapter_pieces_bytes(r, d_in)
    assert nb > 0
    A1, B1, A2, B2 = dev(p["A"]), dev(p["B"]), dev(p["A"]), dev(p["B"])
    p1 = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda")
    p2 = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
    fq.adapter_step(A1, B1, gA, gB, lr)
    fq.adapter_pieces(A1, p1)
    fq.adapter_step_pieces(A2, B2, gA, gB, lr, p2)
    assert np.array_equal(host(A1).view(np.uint32), host(A2).view(np.uint32))
    assert np.array_equal(host(B1).view(np.uint32), host(B2).view(np.uint32))
    h1, h2 = host(p1), host(p2)
    for lo, hi in pieces_regions(r, d_in):
        assert np.array_equal(h1[lo:hi], h2[lo:hi]), (lo, hi)
    if not gpu_lib.melded_linear_xa_fused(T, d_in, d_out, r):
        return
    xq, wq, sx, sw = dev(p["xq"]), dev(p["wq"]), scalar(p["s_x"]), scalar(p["s_w"])
    y1, xa1, y2, xa2 = nan_f32((T, d_out)), nan_f32((T, r)), nan_f32((T, d_out)), nan_f32((T, r))
    fq.melded_linear_fwd_xa(xq, sx, wq, sw, A2, y1, xa1)
    fq.melded_linear_fwd_xa_pieces(xq, sx, wq, sw, p2, r, y2, xa2)
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32))
    assert np.array_equal(host(xa1).view(np.uint32), host(xa2).view(np.uint32))


def test_adapter_pieces_encoding(gpu_lib):
    """The pieces themselves (pieces.hpp's format), decoded on the host with
    the oracle's E4M3 decoder: for every row j and 32-element block (position
    d of a 128-wide K step belongs to block 2 bit4(d) + bit6(d)), the scale
    byte is 127 - e with e the largest integer such that the block's largest
    magnitude m satisfies m 2^e <= 448 (0 for an all-zero block), and each
    element v is reproduced by (dec q0 + dec q1 + dec q2) 2^-e to within
    2^-12 |v| + 2^-10 2^-e (three pieces of 3 significant bits, each rounding
    what the earlier ones left; 2^-10 is half the E4M3 subnormal spacing).
    Rows past r hold zero codes and scale byte 127."""
    fq = gpu_lib
    r, d_in = 13, 512
    announce(f"adapter pieces encoding r={r} d_in={d_in}")
    rng = np.random.default_rng(77)
    A = (rng.standard_normal((r, d_in)) * 10.0 ** rng.uniform(-3, 3, (r, d_in))).astype(np.float32)
    A[2] = 0.0                                    # a zero row
    A[5, 128:160] = 0.0                           # (part of) zero blocks
    A[7, 3] = 3.0e5                               # one large element in its block
    nb = fq.adapter_pieces_bytes(r, d_in)
    buf = torch.full((nb,), 0x77, dtype=torch.uint8, device="cuda")
    fq.adapter_pieces(dev(A), buf)
    h = host(buf)
    rp = (r + 15) // 16 * 16
    (p_lo, p_hi), (e_lo, e_hi) = pieces_regions(r, d_in)
    planes = h[p_lo:p_hi].reshape(3, rp, d_in)
    E = h[e_lo:e_hi].reshape(d_in // 128, rp, 4).astype(np.int64)
    dec = [e4m3.decode(planes[p]).astype(np.float64) for p in range(3)]
    k = np.arange(d_in)
    d = k % 128
    blk = 2 * ((d >> 4) & 1) + ((d >> 6) & 1)                 # block of each column
    c = k // 128
    a64 = A.astype(np.float64)
    for j in range(rp):
        e_col = 127 - E[c, j, blk]                            # the exponent each column sees
        if j >= r:
            assert not planes[:, j].any() and (E[:, j] == 127).all(), j
            continue
        for cc in range(d_in // 128):
            for s in range(4):
                cols = np.nonzero((c == cc) & (blk == s))[0]
                assert cols.size == 32
                m = np.abs(a64[j, cols]).max()
                e = 0 if m == 0 else int(np.floor(np.log2(448.0 / m)))
                if m > 0 and m * 2.0 ** (e + 1) <= 448.0:
                    e += 1                                    # guard log2's rounding both ways
                if m > 0 and m * 2.0 ** e > 448.0:
                    e -= 1
                assert 127 - E[cc, j, s] == e, (j, cc, s, m)
        v_hat = (dec[0][j] + dec[1][j] + dec[2][j]) * np.exp2(-e_col.astype(np.float64))
        bound = 2.0 ** -12 * np.abs(a64[j]) + 2.0 ** -10 * np.exp2(-e_col.astype(np.float64))
        assert (np.abs(v_hat - a64[j]) <= bound).all(), (j, np.max(np.abs(v_hat - a64[j]) / bound))
