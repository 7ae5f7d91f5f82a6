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


def nan_f32(shape):
    """A float32 device tensor filled with NaN: an output element the kernel
    leaves unwritten stays NaN and fails every comparison."""
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def gemm_abs_sum(a_dec, b_dec, s):
    """S[i,j] = sum_k |a_dec[i,k] * b_dec[j,k]| / s in float64: the sum of the
    magnitudes of the products an output element adds up."""
    return (np.abs(a_dec) @ np.abs(b_dec).T) / np.float64(s)


def check_elementwise(got, ref, abs_sum, K, name):
    """Per-element bound on an fp32-accumulated product of K terms each:
        |got - ref| <= (c * S + 4 |ref|) * 2^-24,  c = 2 (ceil(K/128) + 128) + 2
    S = abs_sum: the ordinary error bound of a floating-point sum (each
    addition rounds once, so the error is at most the number of additions on
    any path times 2^-24 times the sum of the magnitudes), counted for a
    128-term dot product per matrix instruction and ceil(K/128) fp32
    accumulations after it, doubled for a truncating adder, plus the scale
    multiply (three roundings) and the float32 rounding of the reference.  A
    missing K block, a transposed operand or an unwritten element exceeds it
    by orders of magnitude."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape == abs_sum.shape, (got.shape, ref.shape, abs_sum.shape)
    c = 2 * (-(-K // 128) + 128) + 2
    bound = (c * abs_sum + 4 * np.abs(ref)) * 2.0 ** -24 + 1e-37
    err = np.abs(got - ref)
    bad = ~(err <= bound)                     # NaN fails
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err / bound, 0))), got.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {got.size} elements outside the "
                             f"per-element bound; worst at {i}: got {got[i]!r}, ref {ref[i]!r}, "
                             f"bound {bound[i]:.3e}")
    return float(np.max(err / bound)) if err.size else 0.0


def rel_l2_rank(g, ref, axis):
    """The largest rel-L2 over the rank components: rows of dA (axis 0) or
    columns of dB (axis 1), so that a wrong small-magnitude component does not
    hide under the large ones."""
    g = np.asarray(g, np.float64)
    ref = np.asarray(ref, np.float64)
    n = g.shape[axis]
    if n == 0:
        return 0.0
    return max(rel_l2(np.take(g, j, axis=axis), np.take(ref, j, axis=axis)) for j in range(n))
