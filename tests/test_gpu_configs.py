"""Parity at the full sizes of the larger workloads, on outputs the oracle can
compute one by one (sampled token rows of Y and dX, sampled rank columns of
dB / rows of dA, sampled backbone rows of the proxy update) and in full where
the oracle is quick enough (quantization codes, r = 64 adapter gradients).

  7B MLP gate projection: W 11008 x 4096, 8192 tokens of bf16 activations;
  13B decoder layer: q (5120 x 5120), up (13824 x 5120), down (5120 x 13824);
  rank sweep: W 4096 x 4096, 8192 tokens, r = 8192 (the largest rank).

Sampling relies on properties of the definitions: a row of Y or dX depends
only on that token's row of X~ or G~; column k of dB depends only on row k of
A, and row k of dA only on column k of B, so the oracle called with A[K] and
B[:, K] gives exactly the ranks K; without a k_max cap a backbone row's score,
selection and new codes depend only on that row.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3
from tests.gpu_util import (TOL, announce, check_elementwise, dev, gemm_bound, host, nan_f32,
                            rel_l2, rel_l2_rank, scalar)
import workloads as wl

pytestmark = pytest.mark.gpu


def quantize(fq, x_np, bf16_bits=None):
    """GPU fp8_quantize of an fp32 array (or of bf16 bit patterns); returns the
    device codes, the device scale, and the host copies."""
    if bf16_bits is not None:
        x = dev(bf16_bits.view(np.int16)).view(torch.bfloat16)
    else:
        x = dev(x_np)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = scalar(0.0)
    fq.fp8_quantize(x, q, s)
    del x
    return q, s, host(q), np.float32(host(s)[0])


def fwd_bwd(fq, tq, ts, xq, xs, gq, gs, A, B):
    T, d_in = xq.shape
    d_out = gq.shape[1]
    r = A.shape[0]
    y = nan_f32((T, d_out))
    fq.melded_linear_fwd(xq, xs, tq, ts, y)
    dx = nan_f32((T, d_in))
    dA = nan_f32((r, d_in))
    dB = nan_f32((d_out, r))
    fq.melded_linear_bwd(gq, gs, xq, xs, tq, ts, dev(A), dev(B), dx, dA, dB)
    return host(y), host(dx), host(dA), host(dB)


def sampled_rows(T, n, seed):
    rows = np.sort(np.random.default_rng(seed).choice(T, n, replace=False))
    return np.unique(np.concatenate([[0], rows, [T - 1]]))


def check_linear(fq, cfg_id, li, spec, rank=None, rank_sample=None, full_grads=True):
    d = wl.make_linear(cfg_id, li, spec, step=0, rank=rank)
    A, B = d["A"], d["B"]
    tw, tsw, wq, s_w = quantize(fq, d["W"])
    rw = oracle.fp8_quantize(d["W"])
    assert np.array_equal(wq, rw[0]) and s_w == rw[1]
    tx, tsx, xq, s_x = quantize(fq, d["X"], d.get("X_bf16"))
    rx = oracle.fp8_quantize(d["X"])            # bf16 widened exactly to fp32
    assert s_x == rx[1]
    assert np.array_equal(xq, rx[0]), "activation codes differ"
    tg, tsg, gq, s_g = quantize(fq, d["dY"])
    rg = oracle.fp8_quantize(d["dY"])
    assert s_g == rg[1] and np.array_equal(gq, rg[0])

    y, dx, dA, dB = fwd_bwd(fq, tw, tsw, tx, tsx, tg, tsg, A, B)
    rows = sampled_rows(spec.tokens, 48, cfg_id * 100 + li)
    ry = oracle.melded_linear_fwd(xq[rows], s_x, wq, s_w)
    rdx, _, _ = oracle.melded_linear_bwd(gq[rows], s_g, xq[rows], s_x, wq, s_w, A[:1], B[:, :1],
                                         want_da=False)
    errs = {"Y": rel_l2(y[rows], ry), "dX": rel_l2(dx[rows], rdx)}
    wd = e4m3.decode(wq)
    check_elementwise(y[rows], ry, gemm_bound(e4m3.decode(xq[rows]), wd,
        np.float64(s_x) * np.float64(s_w), ry), "Y")
    check_elementwise(dx[rows], rdx, gemm_bound(e4m3.decode(gq[rows]), wd.T,
        np.float64(s_g) * np.float64(s_w), rdx), "dX")
    del wd
    assert not np.isnan(dA).any() and not np.isnan(dB).any()
    if full_grads:
        _, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, want_dx=False)
        errs["dA"], errs["dB"] = rel_l2(dA, rdA), rel_l2(dB, rdB)
        errs["dA per rank"], errs["dB per rank"] = rel_l2_rank(dA, rdA, 0), rel_l2_rank(dB, rdB, 1)
    else:
        K = rank_sample
        _, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A[K], B[:, K],
                                               want_dx=False)
        errs["dA"], errs["dB"] = rel_l2(dA[K], rdA), rel_l2(dB[:, K], rdB)
        errs["dA per rank"] = rel_l2_rank(dA[K], rdA, 0)
        errs["dB per rank"] = rel_l2_rank(dB[:, K], rdB, 1)
    print(" ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL, errs
    return d, (tw, tsw, wq, s_w)


def test_mlp_7b_gate_bf16_activations(gpu_lib):
    spec = wl.WORKLOADS[3].linears[0]
    announce(f"7B MLP gate: W {spec.d_out}x{spec.d_in}, T {spec.tokens}, bf16 X, r {spec.rank}")
    check_linear(gpu_lib, 3, 0, spec)


@pytest.mark.parametrize("li", [0, 5, 6])      # q, up, down
def test_decoder_layer_13b_linears(gpu_lib, li):
    spec = wl.WORKLOADS[4].linears[li]
    announce(f"13B {spec.name}: W {spec.d_out}x{spec.d_in}, T {spec.tokens}, r {spec.rank}")
    check_linear(gpu_lib, 4, li, spec)


def test_rank_sweep_largest_rank(gpu_lib):
    """r = 8192 on the 4096 x 4096 backbone with 8192 tokens: fwd/bwd on
    sampled rows and ranks, then the proxy update on sampled backbone rows."""
    spec = wl.WORKLOADS[5].linears[0]
    r = max(wl.RANK_SWEEP)
    announce(f"rank sweep: W 4096x4096, T {spec.tokens}, r {r}")
    K = np.array([0, 1, 777, 4095, 4096, 6000, r - 1])
    d, (tw, tsw, wq, s_w) = check_linear(gpu_lib, 5, 0, spec, rank=r, rank_sample=K,
                                         full_grads=False)
    announce(f"rank sweep proxy update, r {r}, sampled rows")
    A, B = d["A"], d["B"]
    tB = dev(B)
    sel = torch.full((spec.d_out,), -1, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    rho = torch.full((spec.d_out,), np.nan, dtype=torch.float32, device="cuda")
    gpu_lib.rowwise_proxy_update(tw, tsw, dev(A), tB, spec.tau, 0, sel, n, rho=rho)
    g_wq, g_B, g_rho = host(tw), host(tB), host(rho)
    g_sel = host(sel)[: int(host(n)[0])]
    rows = sampled_rows(spec.d_out, 14, 5)
    r_wq, r_B, r_sel, r_rho = oracle.rowwise_proxy_update(wq[rows], s_w, A, B[rows], spec.tau, 0)
    assert np.array_equal(g_rho[rows].view(np.uint32), r_rho.view(np.uint32))
    assert np.array_equal(np.isin(rows, g_sel), np.isin(np.arange(rows.size), r_sel))
    assert np.array_equal(g_wq[rows], r_wq)
    assert np.array_equal(g_B[rows].view(np.uint32), r_B.view(np.uint32))
    print(f"selected {g_sel.size} of {spec.d_out} rows; sampled rows agree bit for bit")
