"""The E5M2 upstream-gradient path on the GPU against the oracle: E5M2 codes,
scale and amax bit-exact (every rounding tie, saturation, NaN); dX, dA, dB
with an E5M2 G~ within rel-L2 1e-3 on the register-staged and the direct-load
GEMM paths; the frozen-A backward; chained steps of the 7B attention
projection with E5M2 gradients."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e5m2
from tests.gpu_util import TOL, announce, dev, host, rel_l2, scalar
from tests.test_oracle_e4m3 import structured_f32_patterns
import workloads as wl

pytestmark = pytest.mark.gpu


def run_q(fq, x_np, dtype="f32", scale_in=None):
    if dtype == "f32":
        x = dev(x_np.astype(np.float32))
    else:
        x = dev(x_np.view(np.int16)).view(torch.bfloat16)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s, amax = scalar(0.0), scalar(0.0)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.fp8_quantize(x, q, s, scale_in=None if scale_in is None else scalar(scale_in), amax=amax,
                    nonfinite=bad, fmt="e5m2")
    return host(q), np.float32(host(s)[0]), np.float32(host(amax)[0]), int(host(bad)[0])


def check_q(fq, x, dtype="f32"):
    q, s, amax, bad = run_q(fq, x, dtype)
    rq, rs, ramax, rbad = oracle.fp8_quantize(x, fmt="e5m2")
    assert s.view(np.uint32) == np.float32(rs).view(np.uint32)
    assert amax.view(np.uint32) == np.float32(ramax).view(np.uint32) and bad == rbad
    mism = np.nonzero(q.ravel() != rq.ravel())[0]
    assert mism.size == 0, f"{mism.size} code mismatches, e.g. idx {mism[:5]}"


def test_e5m2_cast_structured_patterns(gpu_lib):
    """The cast alone (scale 1): every rounding tie of E5M2, one float32 step
    either side, saturation, signed zero, infinities and NaN."""
    announce("E5M2 cast structured patterns, scale 1")
    v = structured_f32_patterns()
    q, _, _, bad = run_q(gpu_lib, v, scale_in=1.0)
    ref = e5m2.encode(v)
    mism = np.nonzero(q != ref)[0]
    assert mism.size == 0, f"{mism.size} mismatches, first {v[mism[:8]]} {q[mism[:8]]} {ref[mism[:8]]}"
    assert bad == int(np.count_nonzero(~np.isfinite(v)))


def test_e5m2_quantize_shapes_and_workload(gpu_lib):
    announce("E5M2 quantize: shapes, bf16, 7B attention dY")
    rng = np.random.default_rng(3)
    for shape in [(256, 512), (257, 33), (1,), (12345,)]:
        check_q(gpu_lib, (rng.standard_normal(shape) * 1e-3).astype(np.float32))
    check_q(gpu_lib, wl.fp32_to_bf16_bits(rng.standard_normal((129, 17)).astype(np.float32)),
            dtype="bf16")
    check_q(gpu_lib, np.zeros(100, np.float32))
    spec = wl.WORKLOADS[2].linears[0]
    check_q(gpu_lib, wl.make_linear(2, 0, spec, step=0)["dY"])


def problem(seed, T, d_in, d_out, r):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    dY = (rng.standard_normal((T, d_out)) * 1e-3).astype(np.float32)
    wq, s_w, _, _ = oracle.fp8_quantize(W)
    xq, s_x, _, _ = oracle.fp8_quantize(X)
    gq, s_g, _, _ = oracle.fp8_quantize(dY, fmt="e5m2")
    A = (rng.standard_normal((r, d_in)) / np.sqrt(r)).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * 1e-3).astype(np.float32)
    return wq, s_w, xq, s_x, gq, s_g, A, B


# K = d_out: 512 and 1024 take the direct-load GEMM (K % 128 == 0), 80 and 272
# the register-staged one; 8320 (65 K steps) splits the dX tiles into two K halves
@pytest.mark.parametrize("T,d_in,d_out,r", [(256, 512, 512, 16), (257, 400, 272, 5),
                                            (600, 1040, 1024, 64), (33, 48, 80, 70),
                                            (256, 1024, 8320, 3)])
def test_e5m2_backward(gpu_lib, T, d_in, d_out, r):
    announce(f"bwd with E5M2 dY: T {T} d_in {d_in} d_out {d_out} r {r}")
    wq, s_w, xq, s_x, gq, s_g, A, B = problem(T + r, T, d_in, d_out, r)
    dx = torch.full((T, d_in), float("nan"), dtype=torch.float32, device="cuda")
    dA = torch.full((r, d_in), float("nan"), dtype=torch.float32, device="cuda")
    dB = torch.full((d_out, r), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_bwd(dev(gq), scalar(s_g), dev(xq), scalar(s_x), dev(wq), scalar(s_w),
                              dev(A), dev(B), dx, dA, dB, g_fmt="e5m2")
    rdx, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, g_fmt="e5m2")
    errs = {"dX": rel_l2(host(dx), rdx), "dA": rel_l2(host(dA), rdA),
            "dB": rel_l2(host(dB), rdB)}
    print(" ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL, errs
    # reading the codes as E4M3 instead would be far off: the format reaches the kernels
    rdx4, _, _ = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, want_da=False)
    assert rel_l2(host(dx), rdx4) > 0.1


def test_e5m2_frozen_backward(gpu_lib):
    announce("frozen-A bwd with E5M2 dY")
    T, d_in, d_out, r = 300, 256, 1024, 13
    wq, s_w, xq, s_x, gq, s_g, A, _ = problem(9, T, d_in, d_out, r)
    aq, s_a, _, _ = oracle.fp8_quantize(A)
    _, u = oracle.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a)
    dx = torch.full((T, d_in), float("nan"), dtype=torch.float32, device="cuda")
    dB = torch.full((d_out, r), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.melded_linear_bwd_frozen_a(dev(gq), scalar(s_g), dev(wq), scalar(s_w), dev(u), dx, dB,
                                       g_fmt="e5m2")
    rdx, rdB = oracle.melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, u, g_fmt="e5m2")
    assert rel_l2(host(dx), rdx) <= TOL and rel_l2(host(dB), rdB) <= TOL


def test_e5m2_chained_steps(gpu_lib):
    """Three steps of the 7B attention projection with E5M2 gradients: codes
    of X, dY and W bit-exact each step; Y, dX, dA, dB within 1e-3; with the
    GPU's gradients the SGD step and the proxy update agree bit for bit."""
    announce("E5M2 dY: 7B attention projection, 3 chained steps")
    spec = wl.WORKLOADS[2].linears[0]
    d0 = wl.make_linear(2, 0, spec, step=0)
    m = gpu_lib.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens, g_fmt="e5m2")
    m.init_state(dev(d0["W"]), dev(d0["A"]), dev(d0["B"]))
    wq, s_w, _, _ = oracle.fp8_quantize(d0["W"])
    A, B = d0["A"], d0["B"]
    for step in range(3):
        d = wl.step_activations(2, 0, spec, step)
        m.step(dev(d["X"]), dev(d["dY"]), lr=spec.lr, tau=spec.tau, k_max=spec.k_max)
        xq, s_x, _, _ = oracle.fp8_quantize(d["X"])
        gq, s_g, _, _ = oracle.fp8_quantize(d["dY"], fmt="e5m2")
        assert np.array_equal(host(m.gq), gq) and host(m.s_g)[0] == s_g
        rows = np.arange(0, spec.tokens, 127)
        rdx, _, _ = oracle.melded_linear_bwd(gq[rows], s_g, xq[rows], s_x, wq, s_w, A[:1],
                                             B[:, :1], want_da=False, g_fmt="e5m2")
        _, rdA, rdB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, want_dx=False,
                                               g_fmt="e5m2")
        gdA, gdB = host(m.dA), host(m.dB)
        errs = (rel_l2(host(m.dx)[rows], rdx), rel_l2(gdA, rdA), rel_l2(gdB, rdB))
        print(f"step {step}: rel-L2 dX {errs[0]:.1e} dA {errs[1]:.1e} dB {errs[2]:.1e}")
        assert max(errs) <= TOL
        A, B = oracle.adapter_step(A, B, gdA, gdB, spec.lr)
        wq, B, sel, _ = oracle.rowwise_proxy_update(wq, s_w, A, B, spec.tau, spec.k_max)
        n_sel = int(host(m.n_sel)[0])
        assert np.array_equal(host(m.sel)[:n_sel], sel)
        assert np.array_equal(host(m.wq), wq)
        assert np.array_equal(host(m.B).view(np.uint32), B.view(np.uint32))
