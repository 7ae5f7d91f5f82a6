"""The backbone's transpose kept across the step: fp8_transpose, the proxy
update that also leaves W~^T (rowwise_proxy_update_t) and the fused backward
that reads it (melded_linear_bwd_xa_t).  Each must give its counterpart's
outputs bit for bit (the plain proxy update and melded_linear_bwd_xa, whose
own parity with the oracle is tested elsewhere), and W~^T must be the exact
transpose of the updated W~."""
import numpy as np
import pytest
import torch

import fp8_quantized_lora_amd as fq_mod
from tests.gpu_util import announce, dev, host, nan_f32, scalar
from tests.test_gpu_linear import quantized_problem
from tests.test_gpu_proxy import proxy_problem
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(16, 16), (272, 400), (4096, 1024), (144, 4096)])
def test_fp8_transpose(gpu_lib, rows, cols):
    announce(f"fp8_transpose {rows} x {cols}")
    rng = np.random.default_rng(rows + cols)
    q = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    qT = torch.full((cols, rows), 0xA5, dtype=torch.uint8, device="cuda")
    gpu_lib.fp8_transpose(dev(q), qT)
    assert np.array_equal(host(qT), q.T)


def _proxy_both(fq, wq, s_w, A, B, tau, k_max):
    d_out, d_in = wq.shape
    out = []
    for keep_t in (False, True):
        twq, tB = dev(wq), dev(B)
        sel = torch.full((d_out,), -1, dtype=torch.int32, device="cuda")
        n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        rho = torch.full((d_out,), np.nan, dtype=torch.float32, device="cuda")
        if keep_t:
            wqT = torch.full((d_in, d_out), 0xA5, dtype=torch.uint8, device="cuda")
            fq.rowwise_proxy_update_t(twq, wqT, scalar(s_w), dev(A), tB, tau, k_max, sel, n,
                                      rho=rho)
        else:
            wqT = None
            fq.rowwise_proxy_update(twq, scalar(s_w), dev(A), tB, tau, k_max, sel, n, rho=rho)
        n_sel = int(host(n)[0])
        out.append((host(twq), host(tB), host(sel)[:n_sel], host(rho),
                    None if wqT is None else host(wqT)))
    return out


@pytest.mark.parametrize("d_out,d_in,r,k_max", [(512, 512, 16, 0), (272, 400, 5, 0),
                                                (1040, 1040, 64, 0), (64, 2048, 130, 0),
                                                (512, 384, 16, 37), (4096, 4096, 64, 0)])
def test_proxy_update_t_matches_and_transposes(gpu_lib, d_out, d_in, r, k_max):
    announce(f"rowwise_proxy_update_t d_out={d_out} d_in={d_in} r={r} k_max={k_max}")
    wq, s_w, A, B = proxy_problem(d_out + d_in + r, d_out, d_in, r)
    (p_wq, p_B, p_sel, p_rho, _), (t_wq, t_B, t_sel, t_rho, t_wqT) = \
        _proxy_both(gpu_lib, wq, s_w, A, B, 0.5, k_max)
    assert 0 < p_sel.size < d_out or k_max, f"fixture merges {p_sel.size} of {d_out} rows"
    assert np.array_equal(t_wq, p_wq) and np.array_equal(t_sel, p_sel)
    assert np.array_equal(t_B.view(np.uint32), p_B.view(np.uint32))
    assert np.array_equal(t_rho.view(np.uint32), p_rho.view(np.uint32))
    assert np.array_equal(t_wqT, t_wq.T), "W~^T is not the transpose of the updated W~"
    print(f"merged {p_sel.size}/{d_out}")


def test_proxy_update_t_nothing_or_everything_merges(gpu_lib):
    """tau above every score (no row merges: W~^T is W~'s transpose as it
    was) and tau = 0 (every row merges)."""
    wq, s_w, A, B = proxy_problem(7, 272, 400, 8)
    for tau in (1e30, 0.0):
        announce(f"rowwise_proxy_update_t tau={tau}")
        (p_wq, p_B, p_sel, _, _), (t_wq, t_B, t_sel, _, t_wqT) = \
            _proxy_both(gpu_lib, wq, s_w, A, B, tau, 0)
        assert p_sel.size == (0 if tau > 1 else 272)
        assert np.array_equal(t_wq, p_wq) and np.array_equal(t_sel, p_sel)
        assert np.array_equal(t_B.view(np.uint32), p_B.view(np.uint32))
        assert np.array_equal(t_wqT, t_wq.T)


BWD_SHAPES = [  # (T, d_in, d_out, r): fused, fused ragged, separate kernels, the large-rank route
    (512, 1024, 1024, 16), (600, 1024, 1280, 16), (257, 400, 272, 5), (1024, 256, 256, 1024),
    (4096, 4096, 4096, 64)]


@pytest.mark.parametrize("T,d_in,d_out,r", BWD_SHAPES)
def test_bwd_xa_t_matches_bwd_xa(gpu_lib, T, d_in, d_out, r):
    announce(f"melded_linear_bwd_xa_t T={T} d_in={d_in} d_out={d_out} r={r}")
    p = quantized_problem(T + r, T, d_in, d_out, r, b_std=0.5)
    xq, wq, A, B = dev(p["xq"]), dev(p["wq"]), dev(p["A"]), dev(p["B"])
    sx, sw, sg = scalar(p["s_x"]), scalar(p["s_w"]), scalar(p["s_g"])
    gq = dev(p["gq"])
    y, xa = nan_f32((T, d_out)), nan_f32((T, r))
    gpu_lib.melded_linear_fwd_xa(xq, sx, wq, sw, A, y, xa)
    wqT = torch.empty((d_in, d_out), dtype=torch.uint8, device="cuda")
    gpu_lib.fp8_transpose(wq, wqT)
    outs = []
    for t in (False, True):
        dx, dA, dB = nan_f32((T, d_in)), nan_f32((r, d_in)), nan_f32((d_out, r))
        if t:
            gpu_lib.melded_linear_bwd_xa_t(gq, sg, xq, sx, wqT, sw, A, B, xa, dx, dA, dB)
        else:
            gpu_lib.melded_linear_bwd_xa(gq, sg, xq, sx, wq, sw, A, B, xa, dx, dA, dB)
        outs.append([host(v).view(np.uint32) for v in (dx, dA, dB)])
    for name, a, b in zip(("dX", "dA", "dB"), *outs):
        assert np.array_equal(a, b), f"{name} differs"


def test_step_keeps_the_transpose(gpu_lib):
    """MeldedLinear with periodic merges keeps W~^T (bwd_xa_t, proxy update
    _t); side by side with the layer that transposes in every backward, over
    four steps that merge every second step, every output and every piece of
    state is the same bit for bit, and the kept W~^T stays W~'s exact
    transpose."""
    spec = wl.LinearSpec("t", d_out=1024, d_in=1024, tokens=512, rank=16, dy_std=1e-2,
                         b_std=1e-3)
    announce("MeldedLinear keeping W~^T vs not, 4 steps, merge every 2nd")
    d = wl.make_linear(11, 0, spec)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    layers = []
    for every in (2, 1):
        m = fq_mod.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens, merge_every=every)
        m.init_state(t(d["W"]), t(d["A"]), t(d["B"]))
        layers.append(m)
    assert layers[0].keep_wt and not layers[1].keep_wt
    merged = 0
    for step in range(4):
        ds = wl.make_linear(11, 0, spec, step=step)
        for m in layers:
            m.forward(t(ds["X"]))
            m.backward(t(ds["dY"]))
            m.update(1e-2, 0.5, merge=step % 2 == 1)
        a, b = layers
        for name in ("y", "dx", "dA", "dB", "A", "B", "wq"):
            x, y = host(getattr(a, name)), host(getattr(b, name))
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (step, name)
        assert np.array_equal(host(a.wqT), host(a.wq).T), step
        if step % 2 == 1:
            merged += int(host(a.n_sel)[0])
    assert merged > 0
