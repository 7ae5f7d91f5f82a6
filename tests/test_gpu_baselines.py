"""The comparison layers on the GPU against the oracle (oracle/baselines.py):
separate-path FP8 LoRA (lora_separate_fp8_fwd / _bwd) and bfloat16 LoRA
(lora_bf16_fwd / _bwd), through the C ABI.

Where a float decides a code -- the E4M3 codes of U = X^ A^^T and V = G^ B^
on the separate path, the bfloat16 values of U and V on the bf16 path -- the
GPU's float32 product and the oracle's exact one can fall on the two sides of
a rounding boundary.  Those codes are compared for what is unique (the
factors' codes and scales bit for bit; U~ and V~ equal except at a small
fraction of elements where the two values are neighbours on the grid), and
the products downstream are checked against the oracle fed the GPU's own
codes (identical inputs), rel-L2 <= 1e-3 as for the melded layer."""
import numpy as np
import pytest
import torch

import oracle
from oracle import baselines as bl
from oracle import e4m3
from tests.gpu_util import (TOL, announce, dev, gemm_bound, host, nan_f32, rel_l2, rel_l2_rank,
                            scalar)

pytestmark = pytest.mark.gpu


def up(v, m):
    return (v + m - 1) // m * m


def problem(seed, T, d_in, d_out, r, b_std=0.5):
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


def codes_valid(got, exact, scale, bound, max_frac, name):
    """E4M3 codes (uint8) of a float32 product quantized with `scale`: equal to
    the codes of the exact product except at a small fraction, and every code
    the nearest-even rounding of some value within `bound` (the per-element
    error bound of the GPU product, gemm_bound) of the exact one."""
    ref = e4m3.encode((exact * np.float64(scale)).astype(np.float32))
    bad = got != ref
    n = int(bad.sum())
    assert n <= max(2, max_frac * got.size), f"{name}: {n} of {got.size} codes differ"
    if n:
        lo = e4m3.decode(e4m3.encode(((exact - bound) * np.float64(scale))[bad].astype(np.float32)))
        hi = e4m3.decode(e4m3.encode(((exact + bound) * np.float64(scale))[bad].astype(np.float32)))
        dg = e4m3.decode(got[bad])
        ok = (lo <= dg) & (dg <= hi)
        assert ok.all(), (name, dg[~ok][:5], lo[~ok][:5], hi[~ok][:5])
    return n


def parse_sep_saved(saved, T, d_in, d_out, r):
    r16 = up(r, 16)
    o = 0
    out = {}
    for name, nbytes in (("aq", r * d_in), ("bq", d_out * r), ("uq", T * r16), ("sc", 16),
                         ("vq", T * r16)):
        out[name] = saved[o:o + nbytes]
        o = up(o + nbytes, 256)
    sc = out["sc"].view(np.float32)
    return dict(aq=out["aq"].reshape(r, d_in), bq=out["bq"].reshape(d_out, r),
                uq=out["uq"].reshape(T, r16), vq=out["vq"].reshape(T, r16),
                s_a=sc[0], s_b=sc[1], s_u=sc[2], s_v=sc[3])


SEP_SHAPES = [(256, 512, 512, 16), (128, 384, 640, 8), (512, 1024, 768, 64),
              (256, 512, 256, 512), (4096, 4096, 4096, 64)]


@pytest.mark.parametrize("T,d_in,d_out,r", SEP_SHAPES)
def test_separate_fp8_parity(gpu_lib, T, d_in, d_out, r):
    announce(f"separate-path FP8 LoRA T={T} d_in={d_in} d_out={d_out} r={r}")
    p = problem(T + r, T, d_in, d_out, r)
    fq = gpu_lib
    xq, wq, gq = dev(p["xq"]), dev(p["wq"]), dev(p["gq"])
    sx, sw, sg = scalar(p["s_x"]), scalar(p["s_w"]), scalar(p["s_g"])
    saved = torch.zeros(fq.lora_separate_fp8_saved_bytes(T, d_in, d_out, r), dtype=torch.uint8,
                        device="cuda")
    y = nan_f32((T, d_out))
    fq.lora_separate_fp8_fwd(xq, sx, wq, sw, dev(p["A"]), dev(p["B"]), y, saved)
    dx, dA, dB = nan_f32((T, d_in)), nan_f32((r, d_in)), nan_f32((d_out, r))
    fq.lora_separate_fp8_bwd(gq, sg, xq, sx, wq, sw, saved, r, dx, dA, dB)
    g = parse_sep_saved(host(saved), T, d_in, d_out, r)
    y, dx, dA, dB = host(y), host(dx), host(dA), host(dB)

    # the factors' codes and scales: bit for bit
    y_ref, sv = bl.lora_separate_fp8_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"], p["A"], p["B"])
    assert np.array_equal(g["aq"], sv["aq"]) and g["s_a"] == sv["s_a"]
    assert np.array_equal(g["bq"], sv["bq"]) and g["s_b"] == sv["s_b"]
    # U~: the scale within a few float32 steps, codes equal but for neighbours
    assert abs(float(g["s_u"]) / float(sv["s_u"]) - 1) < 1e-5
    assert not g["uq"][:, r:].any()
    xd, ad = e4m3.decode(p["xq"]), e4m3.decode(sv["aq"])
    s_xa = np.float64(p["s_x"]) * np.float64(sv["s_a"])
    u64 = xd @ ad.T / s_xa
    nu = codes_valid(g["uq"][:, :r], u64, g["s_u"], gemm_bound(xd, ad, s_xa, u64), 1e-2, "U~")
    # Y against the oracle fed the GPU's U~
    sv_gpu = dict(sv, uq=np.ascontiguousarray(g["uq"][:, :r]), s_u=g["s_u"])
    y0 = oracle.melded_linear_fwd(p["xq"], p["s_x"], p["wq"], p["s_w"])
    lora = bl.fp8_product(sv_gpu["uq"], g["s_u"], sv["bq"], sv["s_b"])
    y_id = (y0.astype(np.float64) + lora).astype(np.float32)
    assert np.linalg.norm(lora) > 0.3 * np.linalg.norm(y0)       # the branch matters
    ey = rel_l2(y, y_id)
    # backward from the GPU's saved codes (V~ too)
    rdx, rdA, rdB, rvq, rsv, _ = bl.lora_separate_fp8_bwd(p["gq"], p["s_g"], p["xq"], p["s_x"],
                                                          p["wq"], p["s_w"], sv_gpu)
    assert abs(float(g["s_v"]) / float(rsv) - 1) < 1e-5
    assert not g["vq"][:, r:].any()
    gd, bdt = e4m3.decode(p["gq"]), e4m3.decode(sv["bq"]).T
    s_gb = np.float64(p["s_g"]) * np.float64(sv["s_b"])
    v64 = gd @ bdt.T / s_gb
    nv = codes_valid(g["vq"][:, :r], v64, g["s_v"], gemm_bound(gd, bdt, s_gb, v64), 1e-2, "V~")
    idx, idA, idB, _, _, _ = bl.lora_separate_fp8_bwd(
        p["gq"], p["s_g"], p["xq"], p["s_x"], p["wq"], p["s_w"], sv_gpu,
        vq=np.ascontiguousarray(g["vq"][:, :r]), s_v=g["s_v"])
    e = (ey, rel_l2(dx, idx), rel_l2(dA, idA), rel_l2(dB, idB), rel_l2_rank(dA, idA, 0),
         rel_l2_rank(dB, idB, 1))
    print("sep FP8 rel-L2 Y %.2e dX %.2e dA %.2e dB %.2e (per rank %.2e %.2e); "
          "U~ / V~ codes off by one step: %d / %d" % (e + (nu, nv)))
    assert max(e) <= TOL


BF16_SHAPES = [(256, 512, 512, 16), (128, 384, 640, 8), (512, 1024, 768, 64),
               (256, 512, 256, 512)]


@pytest.mark.parametrize("T,d_in,d_out,r", BF16_SHAPES)
def test_bf16_lora_parity(gpu_lib, T, d_in, d_out, r):
    announce(f"bf16 LoRA T={T} d_in={d_in} d_out={d_out} r={r}")
    p = problem(T + r + 1, T, d_in, d_out, r)
    fq = gpu_lib
    r64 = up(r, 64)
    X, dY = dev(p["X"]), dev(p["dY"])
    xq, wq, gq = dev(p["xq"]), dev(p["wq"]), dev(p["gq"])
    sx, sw, sg = scalar(p["s_x"]), scalar(p["s_w"]), scalar(p["s_g"])
    saved = torch.zeros(fq.lora_bf16_saved_bytes(T, d_in, d_out, r), dtype=torch.uint8,
                        device="cuda")
    y = nan_f32((T, d_out))
    fq.lora_bf16_fwd(X, xq, sx, wq, sw, dev(p["A"]), dev(p["B"]), y, saved)
    dx, dA, dB = nan_f32((T, d_in)), nan_f32((r, d_in)), nan_f32((d_out, r))
    fq.lora_bf16_bwd(dY, gq, sg, X, wq, sw, dev(p["A"]), dev(p["B"]), saved, dx, dA, dB)
    ub = host(saved).view(np.uint16).reshape(T, r64)
    y, dx, dA, dB = host(y), host(dx), host(dA), host(dB)
    y_ref, ub_ref = bl.lora_bf16_fwd(p["X"], p["xq"], p["s_x"], p["wq"], p["s_w"], p["A"], p["B"])
    assert not ub[:, r:].any()
    u_gpu = (ub[:, :r].astype(np.uint32) << 16).view(np.float32)
    d = np.abs(u_gpu.view(np.int32).astype(np.int64) - ub_ref.view(np.int32).astype(np.int64))
    assert np.all(d[d > 0] == 1 << 16) and (d > 0).mean() <= 1e-2      # neighbours only
    e_y = rel_l2(y, y_ref)
    rdx, rdA, rdB, _ = bl.lora_bf16_bwd(p["dY"], p["gq"], p["s_g"], p["X"], p["wq"], p["s_w"],
                                        p["A"], p["B"], u_gpu)
    e = (e_y, rel_l2(dx, rdx), rel_l2(dA, rdA), rel_l2(dB, rdB), rel_l2_rank(dA, rdA, 0),
         rel_l2_rank(dB, rdB, 1))
    print("bf16 LoRA rel-L2 Y %.2e dX %.2e dA %.2e dB %.2e (per rank %.2e %.2e); U values off "
          "by one bf16 step: %d" % (e + (int((d > 0).sum()),)))
    assert max(e) <= TOL


def test_baselines_reject_unsupported_shapes(gpu_lib):
    announce("baseline shape checks")
    assert gpu_lib.lora_separate_fp8_saved_bytes(100, 64, 64, 8) == 0       # T % 16
    assert gpu_lib.lora_separate_fp8_saved_bytes(128, 64, 64, 12) == 0      # r % 8
    assert gpu_lib.lora_bf16_workspace_bytes(96, 128, 128, 8) == 0          # T % 64
    assert gpu_lib.lora_bf16_workspace_bytes(128, 96, 128, 8) == 0          # d_in % 64
