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


def _group_exp_max(dec, e_min):
    """Per row, per aligned block of 8 consecutive K positions: the largest
    2^e over the block, e the unbiased exponent of each element's code:
    floor(log2 |v|) for normal values, the format's smallest normal exponent
    e_min for subnormals and zeros."""
    a = np.abs(np.asarray(dec, np.float64))
    n, K = a.shape
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** e_min)))
    e = np.maximum(e, e_min)
    pad = (-K) % 8
    if pad:
        e = np.concatenate([e, np.full((n, pad), float(e_min))], axis=1)
    return np.exp2(e.reshape(n, -1, 8).max(axis=2))


def gemm_bound(a_dec, b_dec, s, ref, a_emin=-6, b_emin=-6):
    """Per-element bound on |gpu - ref| for C = a_dec b_dec^T / s computed on
    the gfx950 FP8 matrix cores.  Probed on the hardware (16x16x128 and
    32x32x64 FP8 MFMA): the products of each aligned block of 8 consecutive K
    positions are aligned to the block's largest exponent sum E = max(e_a +
    e_b) and truncated toward zero to multiples of 2^(E-13); the block sums
    then add as in fp32.  The product with exponent sum E has at most 6
    fraction bits and is exact, so a block is off by less than 7 * 2^(E-13)
    <= 7 * 2^-13 * MA * MB (MA, MB: the block's largest 2^e of each operand).
    So, per element,
        |gpu - ref| <= [7 * 2^-13 * sum_blocks MA*MB + (K/8 + 2) 2^-24 S] / s
                       + 4 * 2^-24 |ref|
    with S = sum_k |a_k b_k| (fp32 additions of the block sums and the
    accumulator, the scale multiply (three roundings) and the float32
    rounding of the reference).  a_emin, b_emin: the smallest normal exponent
    of each operand's format (-6 for E4M3, -14 for E5M2)."""
    a_dec = np.asarray(a_dec, np.float64)
    b_dec = np.asarray(b_dec, np.float64)
    K = a_dec.shape[1]
    S = np.abs(a_dec) @ np.abs(b_dec).T
    MM = _group_exp_max(a_dec, a_emin) @ _group_exp_max(b_dec, b_emin).T
    return ((7 * 2.0 ** -13) * MM + (K / 8 + 2) * 2.0 ** -24 * S) / np.float64(s) \
        + 4 * 2.0 ** -24 * np.abs(np.asarray(ref, np.float64))


def check_elementwise(got, ref, bound, name):
    """Every element within its bound (gemm_bound); NaN fails.  Returns the
    largest |got - ref| / bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape == bound.shape, (got.shape, ref.shape, bound.shape)
    bound = bound + 1e-37
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if bad.any():
        ratio = np.where(bad, np.nan_to_num(err / bound, nan=np.inf), -np.inf)
        i = np.unravel_index(int(np.argmax(ratio)), got.shape)
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
