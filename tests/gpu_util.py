"""Helpers shared by the GPU parity tests (device transfer, comparison)."""
import numpy as np
import torch


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def scalar(v, dtype=torch.float32):
    return torch.tensor([v], dtype=dtype, device="cuda")


def rel_l2(x, ref):
    """||x - ref|| / ||ref|| in float64; a zero reference demands an exact zero."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        return 0.0 if not np.any(x) else np.inf
    return float(np.linalg.norm(x - ref) / nr)


TOL = 1e-3   # rel-L2 bound for the fp32-accumulated outputs (Y, dX, dA, dB)


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
