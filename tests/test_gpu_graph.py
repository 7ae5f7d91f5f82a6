"""A whole melded-linear step captured in a HIP graph and replayed gives the
same bits as the same steps run eagerly (every kernel is deterministic and
the step records no memset nodes).  Replays are interleaved with eager work
and synchronisations, and every replay is checked."""
import numpy as np
import pytest
import torch

from tests.gpu_util import announce, dev, host
import workloads as wl

pytestmark = pytest.mark.gpu


def state(m):
    ts = [m.wq, m.A, m.B, m.y, m.dx, m.dB, m.rho]
    ts += [t for t in (m.dA, getattr(m, "u", None), getattr(m, "mB", None),
                       getattr(m, "vB", None), getattr(m, "adam_state", None)) if t is not None]
    return [host(t).copy() for t in ts] + [host(m.sel)[:int(host(m.n_sel)[0])].copy()]


# the default step (A trained, SGD, E4M3), and the pages' own setup: A frozen in
# FP8 (X~A~^T formed in the forward GEMM), 32-bit AdamW whose step count lives
# on the device, and here an E5M2 gradient
CONFIGS = {"default": {}, "frozen_fp8_a_adamw_e5m2": dict(fp8_a=True, optimizer="adamw",
                                                          g_fmt="e5m2"),
           "split_k_halves": {}}
# 8192 features: K = 8192 in both FP8 products, so their 256 x 256 tiles
# (96 in each) run as two K halves added into a zeroed output
SHAPES = {"split_k_halves": (8192, 8192)}


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
def test_graph_replay_matches_eager(gpu_lib, cfg):
    announce(f"graph capture of one step ({cfg}), 3 replays vs eager")
    d_out, d_in = SHAPES.get(cfg, (1024, 1024))
    spec = wl.LinearSpec("g", d_out=d_out, d_in=d_in, tokens=640, rank=16, dy_std=1e-2)
    d = wl.make_linear(7, 0, spec)
    batches = [wl.step_activations(7, 0, spec, s) for s in range(3)]
    mk = lambda: gpu_lib.MeldedLinear(spec.d_out, spec.d_in, spec.rank, spec.tokens,  # noqa: E731
                                      **CONFIGS[cfg])
    eager, graphed = mk(), mk()
    for m in (eager, graphed):
        m.init_state(dev(d["W"]), dev(d["A"]), dev(d["B"]))
    X = dev(batches[0]["X"])
    dY = dev(batches[0]["dY"])
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    # the capture records the launches; the captured step has not run yet
    snapshot = state(graphed)
    with torch.cuda.graph(g, stream=s):
        graphed.step(X, dY, lr=1e-3, tau=0.5)
    torch.cuda.synchronize()
    assert all(np.array_equal(a, b) for a, b in zip(snapshot[:3], state(graphed)[:3]))

    for it in range(3):
        X.copy_(dev(batches[it]["X"]))
        dY.copy_(dev(batches[it]["dY"]))
        eager.step(X, dY, lr=1e-3, tau=0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e, r = state(eager), state(graphed)
        for k, (a, b) in enumerate(zip(e, r)):
            assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
                f"replay {it}: tensor {k} differs"
