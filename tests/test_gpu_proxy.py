"""rowwise_proxy_update on the GPU against the oracle: new codes, new B,
scores, selected rows and their count all bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import announce, dev, host, scalar
import workloads as wl

pytestmark = pytest.mark.gpu


def proxy_problem(seed, d_out, d_in, r, b_scale=0.004, a_std=None):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    wq, s_w, _, _ = oracle.fp8_quantize(W)
    A = (rng.standard_normal((r, d_in)) * (a_std or 1.0 / np.sqrt(max(r, 1)))).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * b_scale).astype(np.float32)
    if d_out:
        B *= rng.choice(np.array([0.05, 0.5, 1.0, 3.0], np.float32), size=(d_out, 1))
    return wq, np.float32(s_w), A, B


def run_gpu(fq, wq, s_w, A, B, tau, k_max):
    d_out = wq.shape[0]
    twq, tB = dev(wq), dev(B)
    sel = torch.full((d_out,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rho = torch.full((d_out,), np.nan, dtype=torch.float32, device="cuda")
    fq.rowwise_proxy_update(twq, scalar(s_w), dev(A), tB, tau, k_max, sel, n, rho=rho)
    n_sel = int(host(n)[0])
    return host(twq), host(tB), host(sel)[:n_sel], host(rho)


def check(fq, wq, s_w, A, B, tau=0.5, k_max=0, expect_some=True):
    g_wq, g_B, g_sel, g_rho = run_gpu(fq, wq, s_w, A, B, tau, k_max)
    r_wq, r_B, r_sel, r_rho = oracle.rowwise_proxy_update(wq, s_w, A, B, tau, k_max)
    assert np.array_equal(g_rho.view(np.uint32), r_rho.view(np.uint32)), \
        f"rho differs at rows {np.nonzero(g_rho != r_rho)[0][:8]}"
    assert np.array_equal(g_sel, r_sel), (g_sel[:10], r_sel[:10])
    bad = np.nonzero(g_wq != r_wq)
    assert bad[0].size == 0, f"{bad[0].size} code mismatches at rows {np.unique(bad[0])[:8]}"
    assert np.array_equal(g_B.view(np.uint32), r_B.view(np.uint32))
    if expect_some:
        assert 0 < r_sel.size, "fixture selects nothing"
    return r_sel


@pytest.mark.parametrize("d_out,d_in,r", [(512, 512, 16), (272, 400, 5), (9, 16, 1),
                                          (1000, 1040, 64), (64, 2048, 130)])
def test_proxy_parity(gpu_lib, d_out, d_in, r):
    announce(f"proxy d_out={d_out} d_in={d_in} r={r}")
    wq, s_w, A, B = proxy_problem(d_out + r, d_out, d_in, r)
    sel = check(gpu_lib, wq, s_w, A, B)
    print(f"selected {sel.size}/{d_out}")


def test_proxy_k_max_and_ties(gpu_lib):
    announce("proxy k_max cap with tied scores")
    wq, s_w, A, B = proxy_problem(7, 300, 256, 8)
    for i in (40, 41, 200, 299):        # four identical rows with the top score
        wq[i] = wq[3]
        B[i] = B[3] * np.float32(30.0)
    B[3] *= np.float32(30.0)
    for k in (1, 2, 3, 5, 17, 299, 300, 1000):
        check(gpu_lib, wq, s_w, A, B, tau=0.5, k_max=k)
    check(gpu_lib, wq, s_w, A, B, tau=0.0, k_max=2)


def test_proxy_limits(gpu_lib):
    announce("proxy tau=inf, tau=0, B=0, r=0, d_out=0")
    wq, s_w, A, B = proxy_problem(8, 200, 128, 4)
    check(gpu_lib, wq, s_w, A, B, tau=np.inf, expect_some=False)
    check(gpu_lib, wq, s_w, A, B, tau=0.0)
    check(gpu_lib, wq, s_w, A, np.zeros_like(B), tau=0.5, expect_some=False)
    check(gpu_lib, wq, s_w, A[:0], B[:, :0], tau=0.0)          # r = 0: -0 codes become +0
    check(gpu_lib, wq[:0], s_w, A, B[:0], tau=0.5, expect_some=False)
    big = B.copy()
    big[::7] = 1e4                                              # saturating merges
    check(gpu_lib, wq, s_w, A, big, tau=0.5)


def test_proxy_full_size_attention_projection(gpu_lib):
    """4096 x 4096 backbone, r = 64, A ~ N(0, 1/r) (variance), B ~ N(0, 1e-3):
    every row scored and merged exactly as the oracle does."""
    announce("proxy full size 4096 x 4096 r=64")
    spec = wl.WORKLOADS[2].linears[0]
    d = wl.make_linear(2, 0, spec)
    wq, s_w, _, _ = oracle.fp8_quantize(d["W"])
    sel = check(gpu_lib, wq, np.float32(s_w), d["A"], d["B"])
    print(f"selected {sel.size}/4096")


def test_proxy_large_rank(gpu_lib):
    announce("proxy 1024 x 4096, r=2048")
    wq, s_w, A, B = proxy_problem(13, 1024, 4096, 2048, b_scale=0.0005)
    check(gpu_lib, wq, s_w, A, B)


@pytest.mark.parametrize("r", [5, 8, 9])
def test_proxy_signed_zero_accumulators(gpu_lib, r):
    """Rows whose every product underflows to -0 end the chain at -0, so
    their -0 codes (0x80) stay -0 when merged (dec + t = -0 + -0); ranks that
    pad the chain to a whole stage on the GPU must not turn such an
    accumulator into +0.  tau = 0 merges every row."""
    announce(f"proxy signed-zero accumulators r={r}")
    rng = np.random.default_rng(100 + r)
    d_out, d_in = 72, 48
    wq = rng.integers(0, 0x7F, size=(d_out, d_in)).astype(np.uint8)
    wq[rng.random(wq.shape) < 0.3] = 0x80
    wq[rng.random(wq.shape) < 0.1] = 0x00
    A = (rng.uniform(1.0, 2.0, (r, d_in)) * 1e-20).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * 1e-3).astype(np.float32)
    B[::2] = (-rng.uniform(1.0, 2.0, (d_out // 2, r)) * 1e-30).astype(np.float32)
    r_wq = oracle.rowwise_proxy_update(wq, np.float32(0.01), A, B, 0.0, 0)[0]
    assert np.count_nonzero(r_wq[::2] == 0x80) > 0, "fixture keeps no -0 code"
    check(gpu_lib, wq, np.float32(0.01), A, B, tau=0.0)


@pytest.mark.parametrize("k_max", [0, 4999])
def test_proxy_many_rows_global_scores(gpu_lib, k_max):
    """d_out = 20001 rows (more than the 16384 scores the selection keeps in
    LDS, so they go through global memory) with a small d_in: codes, B,
    scores and the selection bit-exact, with and without the k_max cap, and
    with no rho output (the scores then live in the workspace)."""
    announce(f"proxy d_out=20001 d_in=32 r=16 k_max={k_max}")
    wq, s_w, A, B = proxy_problem(31 + k_max, 20001, 32, 16)
    sel = check(gpu_lib, wq, s_w, A, B, k_max=k_max)
    assert k_max == 0 or sel.size == k_max
    d_out = wq.shape[0]
    twq, tB = dev(wq), dev(B)
    gsel = torch.full((d_out,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    gpu_lib.rowwise_proxy_update(twq, scalar(s_w), dev(A), tB, 0.5, k_max, gsel, n, rho=None)
    r_wq, r_B, r_sel, _ = oracle.rowwise_proxy_update(wq, s_w, A, B, 0.5, k_max)
    assert np.array_equal(host(gsel)[: int(host(n)[0])], r_sel)
    assert np.array_equal(host(twq), r_wq)
    assert np.array_equal(host(tB).view(np.uint32), r_B.view(np.uint32))
    print(f"selected {sel.size}/{d_out}")
