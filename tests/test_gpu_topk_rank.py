"""rowwise_proxy_update_topk_rank on the GPU against the oracle: the selected
rank components, the selected rows, rho, the merged codes and B bit-exact
(the component scores are maxima, exact on both sides; the chain over the
selected components is the same fixed fmaf order)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import announce, dev, host, scalar
import workloads as wl

pytestmark = pytest.mark.gpu


def run(fq, wq, s_w, A, B, k_rank, tau, k_max=0):
    d_out = wq.shape[0]
    twq, tB = dev(wq), dev(B)
    sel = torch.full((d_out,), -1, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    rho = torch.full((d_out,), float("nan"), dtype=torch.float32, device="cuda")
    K = torch.empty(k_rank, dtype=torch.int32, device="cuda")
    fq.rowwise_proxy_update_topk_rank(twq, scalar(s_w), dev(A), tB, k_rank, tau, k_max, sel, n, K,
                                      rho=rho)
    n_sel = int(host(n)[0])
    return host(twq), host(tB), host(sel)[:n_sel], host(rho), host(K)


def check(fq, wq, s_w, A, B, k_rank, tau, k_max=0):
    g = run(fq, wq, s_w, A, B, k_rank, tau, k_max)
    r_wq, r_B, r_sel, r_rho, r_K = oracle.rowwise_proxy_update_topk_rank(wq, s_w, A, B, k_rank,
                                                                         tau, k_max)
    assert np.array_equal(g[4], r_K), (g[4], r_K)
    assert np.array_equal(g[2], r_sel)
    assert np.array_equal(g[3].view(np.uint32), r_rho.view(np.uint32))
    assert np.array_equal(g[0], r_wq)
    assert np.array_equal(g[1].view(np.uint32), r_B.view(np.uint32))
    return r_sel.size


def problem(seed, d_out, d_in, r, b_scale=1e-3):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    wq, s_w, _, _ = oracle.fp8_quantize(W)
    A = (rng.standard_normal((r, d_in)) / np.sqrt(r)).astype(np.float32)
    # components of very different sizes, so that the choice of K matters
    B = (rng.standard_normal((d_out, r)) * b_scale * 10.0 ** rng.uniform(-1.5, 0.5, r)
         ).astype(np.float32)
    return wq, s_w, A, B


# r > 1024 takes the three-kernel selection (scores, ranks, compaction)
@pytest.mark.parametrize("d_out,d_in,r,k", [(256, 512, 16, 4), (300, 48, 7, 3), (512, 256, 64, 64),
                                             (128, 128, 300, 17), (96, 64, 5, 0),
                                             (160, 64, 2100, 101)])
def test_topk_rank_bit_exact(gpu_lib, d_out, d_in, r, k):
    announce(f"proxy update top-{k} of r {r}: {d_out} x {d_in}")
    wq, s_w, A, B = problem(d_out + r + k, d_out, d_in, r)
    n = check(gpu_lib, wq, s_w, A, B, k, 0.5)
    print(f"selected {n} rows")


def test_topk_rank_ties_and_row_cap(gpu_lib):
    announce("proxy update top-k rank: tied components, k_max cap")
    wq, s_w, A, B = problem(11, 384, 256, 12)
    A[7] = A[2]
    B[:, 7] = B[:, 2]          # components 2 and 7 tie: the lower index is kept
    check(gpu_lib, wq, s_w, A, B, 5, 0.25, k_max=40)
    check(gpu_lib, wq, s_w, A, B, 1, 0.25)


def test_topk_rank_attention_projection(gpu_lib):
    """7B attention projection (4096 x 4096, r = 64), top 16 components."""
    announce("proxy update top-16 of 64: 4096 x 4096")
    spec = wl.WORKLOADS[2].linears[0]
    d = wl.make_linear(2, 0, spec, step=0)
    wq, s_w, _, _ = oracle.fp8_quantize(d["W"])
    B = (d["B"] * np.float32(4.0)).astype(np.float32)    # a few steps' worth of pending delta
    n = check(gpu_lib, wq, s_w, d["A"], B, 16, spec.tau)
    print(f"selected {n} of {spec.d_out} rows")
