"""The frozen-FP8-A calls on the GPU against the oracle: fp8_dequantize bit-exact;
melded_linear_fwd_frozen_a (Y, U) and melded_linear_bwd_frozen_a (dX, dB) within
rel-L2 1e-3 (fp32 accumulation); and chained steps of the pages' training setup
(A frozen in FP8, B trained, proxy update with DQ(A~)) through MeldedLinear."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, announce, dev, host, rel_l2, scalar
import workloads as wl

pytestmark = pytest.mark.gpu


def problem(seed, T, d_in, d_out, r):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    dY = (rng.standard_normal((T, d_out)) * 1e-2).astype(np.float32)
    A = (rng.standard_normal((r, d_in)) / np.sqrt(max(r, 1))).astype(np.float32)
    q = {}
    for name, v in (("w", W), ("x", X), ("g", dY), ("a", A)):
        q[name], q["s_" + name], _, _ = oracle.fp8_quantize(v)
    return q


def test_dequantize_bit_exact(gpu_lib):
    announce("fp8_dequantize")
    rng = np.random.default_rng(1)
    for n, s in ((1000 * 16 + 7, 448.0 / 3.1), (16, 1.0), (5, 0.37), (0, 2.0)):
        codes = rng.integers(0, 256, n).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x11                      # no NaN codes
        q = dev(codes)
        out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        gpu_lib.fp8_dequantize(q, scalar(np.float32(s)), out)
        ref = oracle.fp8_dequantize(codes, np.float32(s))
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32)), n


# the forward forms U inside the FP8 GEMM when d_in % 128 == 0 and the tile
# columns (d_out / 256) number at least 4 * ceil(r / 16): the 4096, (300, 256,
# 1024, 13), (512, 384, 2048, 32) and (200, 128, 1040, 16) cases; the others
# take the separate kernels
@pytest.mark.parametrize("T,d_in,d_out,r", [(256, 512, 512, 16), (777, 48, 80, 5),
                                            (300, 128, 64, 70), (300, 256, 1024, 13),
                                            (512, 384, 2048, 32), (200, 128, 1040, 16),
                                            (4096, 4096, 4096, 64), (4096, 5120, 5120, 64)])
def test_frozen_fwd_bwd(gpu_lib, T, d_in, d_out, r):
    announce(f"frozen-A fwd/bwd T {T} d_in {d_in} d_out {d_out} r {r}")
    q = problem(T + d_in + r, T, d_in, d_out, r)
    xq, wq, gq, aq = dev(q["x"]), dev(q["w"]), dev(q["g"]), dev(q["a"])
    s_x, s_w, s_g, s_a = (scalar(q[k]) for k in ("s_x", "s_w", "s_g", "s_a"))
    y = torch.full((T, d_out), float("nan"), dtype=torch.float32, device="cuda")
    u = torch.full((T, r), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a, y, u)
    dx = torch.full((T, d_in), float("nan"), dtype=torch.float32, device="cuda")
    dB = torch.full((d_out, r), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, u, dx, dB)
    if T * d_in * d_out > 1 << 30:          # large: sampled rows of Y, U and dX
        rows = np.unique(np.concatenate([[0, T - 1],
                                         np.random.default_rng(2).choice(T, 40, replace=False)]))
        ry, ru = oracle.melded_linear_fwd_frozen_a(q["x"][rows], q["s_x"], q["w"], q["s_w"],
                                                   q["a"], q["s_a"])
        rdx, _ = oracle.melded_linear_bwd_frozen_a(q["g"][rows], q["s_g"], q["w"], q["s_w"],
                                                   ru)
        _, ru_full = oracle.melded_linear_fwd_frozen_a(q["x"], q["s_x"], q["w"][:16], q["s_w"],
                                                       q["a"], q["s_a"])
        _, rdB = oracle.melded_linear_bwd_frozen_a(q["g"], q["s_g"], q["w"], q["s_w"], ru_full,
                                                   want_dx=False)
        errs = {"Y": rel_l2(host(y)[rows], ry), "U": rel_l2(host(u)[rows], ru),
                "dX": rel_l2(host(dx)[rows], rdx), "U(all)": rel_l2(host(u), ru_full),
                "dB": rel_l2(host(dB), rdB)}
    else:
        ry, ru = oracle.melded_linear_fwd_frozen_a(q["x"], q["s_x"], q["w"], q["s_w"], q["a"],
                                                   q["s_a"])
        rdx, rdB = oracle.melded_linear_bwd_frozen_a(q["g"], q["s_g"], q["w"], q["s_w"], ru)
        errs = {"Y": rel_l2(host(y), ry), "U": rel_l2(host(u), ru), "dX": rel_l2(host(dx), rdx),
                "dB": rel_l2(host(dB), rdB)}
    print(" ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL, errs


def test_frozen_forward_y_is_the_plain_forward_13b(gpu_lib):
    """4096 x 5120 x 5120 (320 output tiles: the last four tile columns run
    as small tiles in a launch of their own): the frozen-A forward's Y is the
    plain forward's Y bit for bit — the tiles that also form X~A~^T run the
    same products in the same order."""
    announce("frozen-A forward vs plain forward, 4096 x 5120 x 5120")
    q = problem(77, 4096, 5120, 5120, 64)
    xq, wq, aq = dev(q["x"]), dev(q["w"]), dev(q["a"])
    s_x, s_w, s_a = (scalar(q[k]) for k in ("s_x", "s_w", "s_a"))
    y = torch.full((4096, 5120), float("nan"), dtype=torch.float32, device="cuda")
    y0 = torch.full((4096, 5120), float("nan"), dtype=torch.float32, device="cuda")
    u = torch.full((4096, 64), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a, y, u)
    gpu_lib.melded_linear_fwd(xq, s_x, wq, s_w, y0)
    assert torch.equal(y.view(torch.int32), y0.view(torch.int32))
    assert not torch.isnan(u).any()


def test_frozen_edge_cases(gpu_lib):
    announce("frozen-A: T = 0, r = 0, dX skipped")
    q = problem(3, 64, 32, 48, 4)
    xq, wq, gq, aq = dev(q["x"]), dev(q["w"]), dev(q["g"]), dev(q["a"])
    s = {k: scalar(q[k]) for k in ("s_x", "s_w", "s_g", "s_a")}
    # no tokens: dB is all zeros
    dB = torch.full((48, 4), np.nan, dtype=torch.float32, device="cuda")
    u0 = torch.full((0, 4), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_bwd_frozen_a(gq[:0], s["s_g"], wq, s["s_w"], u0, None, dB)
    assert not host(dB).any()
    # rank 0: U is empty, Y still computed
    y = torch.full((64, 48), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_fwd_frozen_a(xq, s["s_x"], wq, s["s_w"], aq[:0], s["s_a"], y,
                                       torch.full((64, 0), float("nan"), dtype=torch.float32, device="cuda"))
    assert rel_l2(host(y), oracle.melded_linear_fwd(q["x"], q["s_x"], q["w"], q["s_w"])) <= TOL
    # dX skipped
    u = torch.full((64, 4), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_fwd_frozen_a(xq, s["s_x"], wq, s["s_w"], aq, s["s_a"], y, u)
    gpu_lib.melded_linear_bwd_frozen_a(gq, s["s_g"], wq, s["s_w"], u, None, dB)
    _, rdB = oracle.melded_linear_bwd_frozen_a(q["g"], q["s_g"], q["w"], q["s_w"], host(u),
                                               want_dx=False)
    assert rel_l2(host(dB), rdB) <= TOL


def test_frozen_fp8_a_chained_steps(gpu_lib):
    """Three steps of the 7B attention projection with A frozen in FP8.  The
    oracle takes the GPU's dB for its SGD step (a rel-L2 check covers dB), so
    B, the scores and the merged codes must then agree bit for bit."""
    announce("frozen FP8 A: 7B attention projection, 3 chained steps")
    spec = wl.WORKLOADS[2].linears[0]
    d0 = wl.make_linear(2, 0, spec, step=0)
    m = gpu_lib.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens, fp8_a=True)
    m.init_state(dev(d0["W"]), dev(d0["A"]), dev(d0["B"]))
    wq, s_w, _, _ = oracle.fp8_quantize(d0["W"])
    aq, s_a, _, _ = oracle.fp8_quantize(d0["A"])
    assert np.array_equal(host(m.aq), aq) and host(m.s_a)[0] == s_a
    A = oracle.fp8_dequantize(aq, s_a)
    assert np.array_equal(host(m.A).view(np.uint32), A.view(np.uint32))
    B = d0["B"]
    for step in range(3):
        d = wl.step_activations(2, 0, spec, step)
        m.step(dev(d["X"]), dev(d["dY"]), lr=spec.lr, tau=spec.tau, k_max=spec.k_max)
        xq, s_x, _, _ = oracle.fp8_quantize(d["X"])
        gq, s_g, _, _ = oracle.fp8_quantize(d["dY"])
        rows = np.arange(0, spec.tokens, 97)
        ry, ru = oracle.melded_linear_fwd_frozen_a(xq[rows], s_x, wq, s_w, aq, s_a)
        _, ru_all = oracle.melded_linear_fwd_frozen_a(xq, s_x, wq[:16], s_w, aq, s_a)
        rdx, rdB = oracle.melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, ru_all)
        errs = (rel_l2(host(m.y)[rows], ry), rel_l2(host(m.u), ru_all),
                rel_l2(host(m.dx), rdx), rel_l2(host(m.dB), rdB))
        g_dB = host(m.dB)
        _, B1 = oracle.adapter_step(A, B, None, g_dB, spec.lr)
        wq2, B2, sel, rho = oracle.rowwise_proxy_update(wq, s_w, A, B1, spec.tau, spec.k_max)
        n_sel = int(host(m.n_sel)[0])
        print(f"step {step}: rel-L2 Y {errs[0]:.1e} U {errs[1]:.1e} dX {errs[2]:.1e} "
              f"dB {errs[3]:.1e}; selected {n_sel}/{spec.d_out}")
        assert max(errs) <= TOL
        assert np.array_equal(host(m.sel)[:n_sel], sel)
        assert np.array_equal(host(m.rho).view(np.uint32), rho.view(np.uint32))
        assert np.array_equal(host(m.wq), wq2)
        assert np.array_equal(host(m.B).view(np.uint32), B2.view(np.uint32))
        assert np.array_equal(host(m.A).view(np.uint32), A.view(np.uint32))     # frozen
        wq, B = wq2, B2
