"""Whole steps chained on the GPU (MeldedLinear) against the oracle's chain.

Per call on identical inputs the results are bit-exact (codes, rows) or within
rel-L2 1e-3 (floats); chained over steps, tolerance-level differences in dA/dB
move B, so a row whose score sits at the threshold may flip.  These tests
assert that every differing selection is such a borderline row and that all
other state agrees."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, announce, dev, host, rel_l2
import workloads as wl

pytestmark = pytest.mark.gpu


def oracle_step(st, X, dY, lr, tau, k_max=0):
    xq, s_x, _, _ = oracle.fp8_quantize(X)
    y = oracle.melded_linear_fwd(xq, s_x, st["wq"], st["s_w"])
    gq, s_g, _, _ = oracle.fp8_quantize(dY)
    dx, dA, dB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, st["wq"], st["s_w"], st["A"], st["B"])
    A, B = oracle.adapter_step(st["A"], st["B"], dA, dB, lr)
    wq, B, sel, rho = oracle.rowwise_proxy_update(st["wq"], st["s_w"], A, B, tau, k_max)
    return dict(wq=wq, s_w=st["s_w"], A=A, B=B), dict(y=y, dx=dx, dA=dA, dB=dB, sel=sel, rho=rho)


def run_chain(fq, cfg_id, steps, tol_rows_frac=0.01):
    spec = wl.WORKLOADS[cfg_id].linears[0]
    d0 = wl.make_linear(cfg_id, 0, spec, step=0)
    m = fq.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens)
    m.init_state(dev(d0["W"]), dev(d0["A"]), dev(d0["B"]))
    wq0, s_w, _, _ = oracle.fp8_quantize(d0["W"])
    assert np.array_equal(host(m.wq), wq0)
    st = dict(wq=wq0, s_w=np.float32(s_w), A=d0["A"], B=d0["B"])
    for step in range(steps):
        d = wl.step_activations(cfg_id, 0, spec, step)
        X, dY = dev(d["X"]), dev(d["dY"])
        m.step(X, dY, lr=spec.lr, tau=spec.tau, k_max=spec.k_max)
        st, out = oracle_step(st, d["X"], d["dY"], spec.lr, spec.tau, spec.k_max)
        e = (rel_l2(host(m.y), out["y"]), rel_l2(host(m.dx), out["dx"]),
             rel_l2(host(m.dA), out["dA"]), rel_l2(host(m.dB), out["dB"]))
        n_sel = int(host(m.n_sel)[0])
        g_sel = host(m.sel)[:n_sel]
        flips = np.setxor1d(g_sel, out["sel"])
        rho = out["rho"]
        margin = np.abs(rho[flips] - spec.tau) / spec.tau if flips.size else np.zeros(0)
        code_rows = np.nonzero(np.any(host(m.wq) != st["wq"], axis=1))[0]
        print(f"step {step}: rel-L2 Y {e[0]:.2e} dX {e[1]:.2e} dA {e[2]:.2e} dB {e[3]:.2e}; "
              f"selected {n_sel}/{spec.d_out}, flips {flips.size}, rows with code drift "
              f"{code_rows.size}")
        assert max(e[:2]) <= TOL
        assert e[2] <= TOL and e[3] <= TOL
        assert np.all(margin < 1e-3), (flips, margin)
        assert code_rows.size <= max(1, int(tol_rows_frac * spec.d_out))
        # continue both chains from the GPU's state so that drift does not compound
        st = dict(wq=host(m.wq), s_w=st["s_w"], A=host(m.A), B=host(m.B))


def test_single_linear_step(gpu_lib):
    announce("chained step: 512 x 512 single linear")
    run_chain(gpu_lib, 1, 1)


def test_attention_projection_ten_steps(gpu_lib):
    announce("chained steps: 7B attention projection, 10 steps")
    run_chain(gpu_lib, 2, 10)
