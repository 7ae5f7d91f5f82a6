"""Whole steps chained on the GPU (MeldedLinear) against the oracle's chain.

Per call on identical inputs the results are bit-exact (codes, rows) or within
rel-L2 1e-3 (floats).  The float gradients dA, dB agree with the oracle's own
to that bound, not bit for bit, and an adapter moved by a rounding-level
amount may legitimately flip a row whose score sits at the threshold or a
merged code whose dec(q) + t sits at a rounding midpoint.  So the oracle's
optimizer takes the GPU's gradients (checked against the oracle's own, rel-L2
<= 1e-3), after which the adapters (and AdamW moments), the row scores, the
selected rows and the backbone codes must agree bit for bit.  Each step
restarts the oracle from the GPU's state, so the comparison does not
compound."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, announce, dev, host, rel_l2
import workloads as wl

pytestmark = pytest.mark.gpu


ADAMW = dict(beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def oracle_step(st, X, dY, lr, tau, k_max=0, opt_step=0, grads=None):
    """One oracle step from state st; with `grads` = (dA, dB) the adapter
    optimizer takes those gradients instead of the oracle's own."""
    xq, s_x, _, _ = oracle.fp8_quantize(X)
    y = oracle.melded_linear_fwd(xq, s_x, st["wq"], st["s_w"])
    gq, s_g, _, _ = oracle.fp8_quantize(dY)
    dx, dA, dB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, st["wq"], st["s_w"], st["A"], st["B"])
    new = {}
    uA, uB = (dA, dB) if grads is None else grads
    if opt_step == 0:
        A, B = oracle.adapter_step(st["A"], st["B"], uA, uB, lr)
    else:
        A, B, mA, vA, mB, vB = oracle.adapter_step_adamw(
            st["A"], st["B"], uA, uB, st["mA"], st["vA"], st["mB"], st["vB"], lr,
            ADAMW["beta1"], ADAMW["beta2"], ADAMW["eps"], ADAMW["weight_decay"], opt_step)
        new = dict(mA=mA, vA=vA, mB=mB, vB=vB)
    _, t = oracle.row_scores(st["wq"], st["s_w"], A, B)
    wq, B, sel, rho = oracle.rowwise_proxy_update(st["wq"], st["s_w"], A, B, tau, k_max)
    return dict(wq=wq, s_w=st["s_w"], A=A, B=B, **new), dict(y=y, dx=dx, dA=dA, dB=dB, sel=sel,
                                                             rho=rho, t=t)


def run_chain(fq, cfg_id, steps, optimizer="sgd"):
    spec = wl.WORKLOADS[cfg_id].linears[0]
    d0 = wl.make_linear(cfg_id, 0, spec, step=0)
    m = fq.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens, optimizer=optimizer,
                        adamw=ADAMW)
    m.init_state(dev(d0["W"]), dev(d0["A"]), dev(d0["B"]))
    wq0, s_w, _, _ = oracle.fp8_quantize(d0["W"])
    assert np.array_equal(host(m.wq), wq0)
    st = dict(wq=wq0, s_w=np.float32(s_w), A=d0["A"], B=d0["B"])
    if optimizer == "adamw":
        st.update(mA=np.zeros_like(d0["A"]), vA=np.zeros_like(d0["A"]),
                  mB=np.zeros_like(d0["B"]), vB=np.zeros_like(d0["B"]))
    for step in range(steps):
        d = wl.step_activations(cfg_id, 0, spec, step)
        m.step(dev(d["X"]), dev(d["dY"]), lr=spec.lr, tau=spec.tau, k_max=spec.k_max)
        grads = (host(m.dA), host(m.dB))
        st, out = oracle_step(st, d["X"], d["dY"], spec.lr, spec.tau, spec.k_max,
                              opt_step=0 if optimizer == "sgd" else step + 1, grads=grads)
        e = (rel_l2(host(m.y), out["y"]), rel_l2(host(m.dx), out["dx"]),
             rel_l2(grads[0], out["dA"]), rel_l2(grads[1], out["dB"]))
        n_sel = int(host(m.n_sel)[0])
        g_sel = host(m.sel)[:n_sel]
        g_wq = host(m.wq)
        print(f"step {step}: rel-L2 Y {e[0]:.2e} dX {e[1]:.2e} dA {e[2]:.2e} dB {e[3]:.2e}; "
              f"selected {n_sel}/{spec.d_out}")
        assert max(e) <= TOL
        assert np.array_equal(g_sel, out["sel"])
        assert np.array_equal(g_wq, st["wq"])
        keys = ("A", "B") + (("mA", "vA", "mB", "vB") if optimizer == "adamw" else ())
        for k in keys:
            assert np.array_equal(host(getattr(m, k)).view(np.uint32), st[k].view(np.uint32)), k
        assert np.array_equal(host(m.rho).view(np.uint32), out["rho"].view(np.uint32))
        st = dict(wq=g_wq, s_w=st["s_w"], A=host(m.A), B=host(m.B))
        if optimizer == "adamw":
            st.update(mA=host(m.mA), vA=host(m.vA), mB=host(m.mB), vB=host(m.vB))


def test_single_linear_step(gpu_lib):
    announce("chained step: 512 x 512 single linear")
    run_chain(gpu_lib, 1, 1)


def test_attention_projection_ten_steps(gpu_lib):
    announce("chained steps: 7B attention projection, 10 steps")
    run_chain(gpu_lib, 2, 10)


def test_attention_projection_adamw_three_steps(gpu_lib):
    announce("chained steps: 7B attention projection, 32-bit AdamW, 3 steps")
    run_chain(gpu_lib, 2, 3, optimizer="adamw")


def test_merge_interval(gpu_lib):
    """Proxy merged every third step (the pages merge the accumulated proxy
    into the backbone periodically): between merges W~ is untouched and B
    accumulates the SGD updates; on merge steps the oracle's proxy update,
    given the GPU's adapter gradients, yields the same rows, codes and B bit
    for bit."""
    announce("merge every 3 steps: 512 x 512 single linear, 6 steps")
    spec = wl.WORKLOADS[1].linears[0]
    d0 = wl.make_linear(1, 0, spec, step=0)
    m = gpu_lib.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens)
    m.init_state(dev(d0["W"]), dev(d0["A"]), dev(d0["B"]))
    wq, s_w, _, _ = oracle.fp8_quantize(d0["W"])
    A, B = d0["A"], d0["B"]
    merged_rows = 0
    for step in range(6):
        d = wl.step_activations(1, 0, spec, step)
        m.step(dev(d["X"]), dev(d["dY"]), lr=spec.lr, tau=spec.tau, k_max=spec.k_max,
               merge_every=3)
        xq, s_x, _, _ = oracle.fp8_quantize(d["X"])
        gq, s_g, _, _ = oracle.fp8_quantize(d["dY"])
        _, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, want_dx=False)
        gdA, gdB = host(m.dA), host(m.dB)
        assert rel_l2(gdA, rdA) <= TOL and rel_l2(gdB, rdB) <= TOL
        A, B = oracle.adapter_step(A, B, gdA, gdB, spec.lr)
        if (step + 1) % 3 == 0:
            wq, B, sel, _ = oracle.rowwise_proxy_update(wq, s_w, A, B, spec.tau, spec.k_max)
            n_sel = int(host(m.n_sel)[0])
            assert np.array_equal(host(m.sel)[:n_sel], sel)
            merged_rows += n_sel
        assert np.array_equal(host(m.wq), wq), step
        assert np.array_equal(host(m.A).view(np.uint32), A.view(np.uint32)), step
        assert np.array_equal(host(m.B).view(np.uint32), B.view(np.uint32)), step
    print(f"rows merged over 2 merges: {merged_rows}")
    assert merged_rows > 0
