"""FP4 E2M1 variant on the GPU against the oracle: fp4_quantize codes, scale
and amax bit-exact (the device encodes with comparisons against the seven
midpoints, the oracle by rounding on the grid spacing); melded_linear_fwd_fp4
within the rel-L2 bound (the products are exact, the fp32 sums are not)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e2m1
from tests.gpu_util import TOL, announce, dev, host, rel_l2, scalar
import workloads as wl

pytestmark = pytest.mark.gpu


def run_quantize(fq, x_np, dtype="f32", scale_in=None):
    if dtype == "f32":
        x = dev(x_np.astype(np.float32))
    else:   # bf16 bit patterns as uint16
        x = dev(x_np.view(np.int16)).view(torch.bfloat16)
    q = torch.empty(tuple(x.shape[:-1]) + (x.shape[-1] // 2,), dtype=torch.uint8, device="cuda")
    s, amax = scalar(0.0), scalar(0.0)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.fp4_quantize(x, q, s, scale_in=None if scale_in is None else scalar(scale_in), amax=amax,
                    nonfinite=bad)
    return host(q), np.float32(host(s)[0]), np.float32(host(amax)[0]), int(host(bad)[0])


def check_quantize(fq, x, dtype="f32", scale_in=None):
    q, s, amax, bad = run_quantize(fq, x, dtype, scale_in)
    rq, rs, ramax, rbad = oracle.fp4_quantize(x, scale_in=scale_in)
    assert s.view(np.uint32) == np.float32(rs).view(np.uint32), (s, rs)
    assert amax.view(np.uint32) == np.float32(ramax).view(np.uint32)
    assert bad == rbad
    mism = np.nonzero(q.ravel() != rq.ravel())[0]
    assert mism.size == 0, f"{mism.size} byte mismatches, e.g. idx {mism[:5]}"
    return rq


@pytest.mark.parametrize("shape", [(256, 512), (257, 34), (1, 2), (5, 2), (12346,), (3, 5, 8)])
def test_fp4_quantize_random_shapes(gpu_lib, shape):
    announce(f"fp4 quantize f32 {shape}")
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * 3.0).astype(np.float32)
    check_quantize(gpu_lib, x)


def test_fp4_quantize_ties_specials_bf16(gpu_lib):
    announce("fp4 quantize: exact midpoints, saturation, NaN/inf, bf16 input")
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9))])
    x = np.concatenate([near, -near, [0.0, -0.0, 6.0, 7.0, 1e30, -1e30, np.inf, -np.inf, np.nan,
                                      0.1, -0.1]]).astype(np.float32)
    x = np.concatenate([x, np.zeros(x.size % 2, np.float32)])
    q = check_quantize(gpu_lib, x, scale_in=1.0)
    c = e2m1.unpack(q)
    assert list(c[:7]) == [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6]      # ties go to the even code
    # bf16 input: the tail of a length not divisible by 8
    rng = np.random.default_rng(9)
    xb = (rng.standard_normal(1000 * 8 + 6) * 2.0).astype(np.float32)
    bits = (xb.view(np.uint32) >> 16).astype(np.uint16)
    check_quantize(gpu_lib, bits, dtype="bf16")


def run_fwd(fq, xq, s_x, wq, s_w):
    T, d_out = xq.shape[0], wq.shape[0]
    y = torch.full((T, d_out), float("nan"), dtype=torch.float32, device="cuda")
    fq.melded_linear_fwd_fp4(dev(xq), scalar(s_x), dev(wq), scalar(s_w), y)
    return host(y)


@pytest.mark.parametrize("T,d_in,d_out", [(256, 256, 256), (300, 512, 272), (1, 256, 16),
                                          (513, 1024, 528),
                                          # 16640 values = 8320 bytes = 65 K steps: both
                                          # tiles run as two K halves (32 and 33 steps)
                                          (256, 16640, 304)])
def test_fp4_forward_parity(gpu_lib, T, d_in, d_out):
    announce(f"fp4 forward T={T} d_in={d_in} d_out={d_out}")
    rng = np.random.default_rng(T + d_in + d_out)
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    xq, s_x, _, _ = oracle.fp4_quantize(X)
    wq, s_w, _, _ = oracle.fp4_quantize(W)
    y = run_fwd(gpu_lib, xq, s_x, wq, s_w)
    ref = oracle.melded_linear_fwd_fp4(xq, s_x, wq, s_w)
    err = rel_l2(y, ref)
    print(f"rel-L2 {err:.2e}")
    assert err <= TOL


def test_fp4_forward_attention_projection(gpu_lib):
    """7B attention projection (X 4096 x 4096 with outlier channels, W 4096 x
    4096), quantized on the GPU; Y checked on sampled token rows (a row of Y
    depends only on that token's row of X~)."""
    announce("fp4 forward 4096 x 4096 x 4096 (sampled rows)")
    spec = wl.WORKLOADS[2].linears[0]
    d = wl.make_linear(2, 0, spec, step=0)
    tx = torch.empty((spec.tokens, spec.d_in // 2), dtype=torch.uint8, device="cuda")
    tw = torch.empty((spec.d_out, spec.d_in // 2), dtype=torch.uint8, device="cuda")
    sx, sw = scalar(0.0), scalar(0.0)
    gpu_lib.fp4_quantize(dev(d["X"]), tx, sx)
    gpu_lib.fp4_quantize(dev(d["W"]), tw, sw)
    y = torch.full((spec.tokens, spec.d_out), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_fwd_fp4(tx, sx, tw, sw, y)
    xq, wq, hy = host(tx), host(tw), host(y)
    rxq, rs_x, _, _ = oracle.fp4_quantize(d["X"])
    rwq, rs_w, _, _ = oracle.fp4_quantize(d["W"])
    assert np.float32(host(sx)[0]) == rs_x and np.float32(host(sw)[0]) == rs_w
    assert np.array_equal(rxq, xq) and np.array_equal(rwq, wq)
    rows = np.unique(np.concatenate([[0, spec.tokens - 1],
                                     np.random.default_rng(1).choice(spec.tokens, 62, replace=False)]))
    ref = oracle.melded_linear_fwd_fp4(xq[rows], rs_x, wq, rs_w)
    err = rel_l2(hy[rows], ref)
    print(f"rel-L2 {err:.2e} over {rows.size} rows")
    assert err <= TOL
