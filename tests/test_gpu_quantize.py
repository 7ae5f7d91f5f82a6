"""fp8_quantize on the GPU against the oracle: codes, scale and amax bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3
from tests.gpu_util import announce, dev, host, scalar
from tests.test_oracle_e4m3 import structured_f32_patterns
import workloads as wl

pytestmark = pytest.mark.gpu


def run_gpu(fq, x_np, dtype="f32", scale_in=None):
    if dtype == "f32":
        x = dev(x_np.astype(np.float32))
    else:   # x_np holds bf16 bit patterns as uint16
        x = dev(x_np.view(np.int16)).view(torch.bfloat16)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = scalar(0.0)
    amax = scalar(0.0)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.fp8_quantize(x, q, s, scale_in=None if scale_in is None else scalar(scale_in), amax=amax,
                    nonfinite=bad)
    return host(q), np.float32(host(s)[0]), np.float32(host(amax)[0]), int(host(bad)[0])


def check(fq, x, dtype="f32", scale_in=None):
    q, s, amax, bad = run_gpu(fq, x, dtype, scale_in)
    rq, rs, ramax, rbad = oracle.fp8_quantize(x, scale_in=scale_in)
    assert s.view(np.uint32) == np.float32(rs).view(np.uint32), (s, rs)
    assert amax.view(np.uint32) == np.float32(ramax).view(np.uint32)
    assert bad == rbad
    mism = np.nonzero(q.ravel() != rq.ravel())[0]
    assert mism.size == 0, f"{mism.size} code mismatches, e.g. idx {mism[:5]}"


@pytest.mark.parametrize("shape", [(256, 512), (257, 33), (1, 1), (12345,), (3, 5, 7), (4096, 16)])
def test_quantize_random_shapes(gpu_lib, shape):
    announce(f"quantize f32 {shape}")
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(3.0)
    check(gpu_lib, x)


def test_quantize_workload_activations(gpu_lib):
    spec = wl.WORKLOADS[2].linears[0]
    announce("quantize 7B attention X with outlier channels (4096 x 4096) and dY")
    d = wl.make_linear(2, 0, spec, step=0)
    check(gpu_lib, d["X"])
    check(gpu_lib, d["dY"])
    check(gpu_lib, d["W"])


def test_quantize_bf16(gpu_lib):
    announce("quantize bf16")
    rng = np.random.default_rng(5)
    for shape in [(8192, 64), (129, 17), (7,)]:
        x = rng.standard_normal(shape).astype(np.float32)
        xb = wl.fp32_to_bf16_bits(x)
        check(gpu_lib, xb, dtype="bf16")


def test_cast_structured_patterns_static_scale(gpu_lib):
    """The cast alone (scale 1): every rounding tie, one float32 step either
    side of it, saturation, signed zero, inf and NaN."""
    announce("cast structured patterns, scale 1")
    v = structured_f32_patterns()
    q, s, amax, bad = run_gpu(gpu_lib, v, scale_in=1.0)
    ref = e4m3.encode(v)
    mism = np.nonzero(q != ref)[0]
    assert mism.size == 0, f"{mism.size} mismatches, first {v[mism[:8]]} {q[mism[:8]]} {ref[mism[:8]]}"
    assert bad == int(np.count_nonzero(~np.isfinite(v)))


def test_quantize_edge_cases(gpu_lib):
    announce("quantize edge cases")
    check(gpu_lib, np.zeros(0, np.float32))
    check(gpu_lib, np.zeros(1000, np.float32))
    check(gpu_lib, np.array([-0.0, 0.0, -0.0, 0.0, -0.0], np.float32))
    check(gpu_lib, np.array([1e-45, -1e-45, 0.0, 1e-45], np.float32))     # scale -> FLT_MAX
    check(gpu_lib, np.array([1.0, np.nan, -2.0, np.inf, 0.5, -np.inf, 3.0], np.float32))
    big = np.full(5000, 3.0e38, np.float32)
    big[17] = -3.4e38
    check(gpu_lib, big)


def test_quantize_is_deterministic(gpu_lib):
    announce("quantize twice, bitwise equal")
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1024, 1024)).astype(np.float32)
    a = run_gpu(gpu_lib, x)
    b = run_gpu(gpu_lib, x)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1]


def test_quantize_double_rounding_golden(gpu_lib):
    """The golden cases whose fl32(x*s) lands exactly on an E4M3 midpoint that
    the exact product misses (tests/golden/fp8_double_rounding.txt, derived on
    exact rationals): the GPU cast gives the fixture's two-rounding code,
    with the scale given and with the scale from the tensor's amax."""
    from tests.test_oracle_linear import load_double_rounding_golden
    announce("quantize double-rounding golden cases")
    rows = load_double_rounding_golden()
    x = np.array([r[0] for r in rows], np.float32)
    s_all = np.array([r[1] for r in rows], np.float32)
    want = np.array([r[2] for r in rows], np.uint8)
    for s in np.unique(s_all):
        k = s_all == s
        q, s_out, _, _ = run_gpu(gpu_lib, x[k], scale_in=s)
        assert s_out == s and np.array_equal(q, want[k]), (s, q, want[k])
    for amax in (np.float32(3.1), np.float32(0.0731)):
        s = np.float32(448.0) / amax
        k = s_all == s
        q, s_out, a_out, _ = run_gpu(gpu_lib, np.concatenate([[amax], x[k]]).astype(np.float32))
        assert s_out == s and a_out == amax and np.array_equal(q[1:], want[k])


def _quantize_dev(fq, x, fmt="e4m3", stream=None):
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s, amax = scalar(0.0), scalar(0.0)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.fp8_quantize(x, q, s, amax=amax, nonfinite=bad, fmt=fmt, stream=stream)
    return q, s, amax, bad


def test_quantize_across_the_one_launch_limit(gpu_lib):
    """x of up to 64 MiB takes the one launch with x in registers, a little
    more the one launch with part of x in LDS: calls alternating between the
    two and between sizes (so the exchange words of the one-launch form hold
    an earlier call's values) all match the oracle bit for bit."""
    rng = np.random.default_rng(31)
    n_one = 4096 * 4096                 # 1024 workgroups: the largest one-launch fp32 x
    for n, seed in [(n_one, 1), (n_one + 4, 2), (3 * 4096 + 5, 3), (n_one, 4), (n_one - 4096, 5)]:
        announce(f"quantize f32 n={n} seed {seed}")
        x = (rng.standard_normal(n) * (seed + 1)).astype(np.float32)
        x[rng.integers(0, n, 3)] = [np.inf, np.nan, -np.inf]
        check(gpu_lib, x)


def test_quantize_across_the_lds_staged_limit(gpu_lib):
    """Above 64 MiB the one launch also stages 9 vectors per lane in LDS (up
    to 1024 workgroups x 25 x 256 vectors = 100 MiB of fp32); one element
    group more takes the two launches.  The 13B layer's 4096 x 5120 fp32
    activations (80 MiB) fall in between.  All bit-exact; one pass with no
    wait, so that the fallback reads ranges of the LDS-staged layout."""
    rng = np.random.default_rng(35)
    n_lds = 1024 * 25 * 256 * 4
    for n in (4096 * 5120, n_lds, n_lds + 4):
        announce(f"quantize f32 n={n} (LDS-staged limit)")
        x = (rng.standard_normal(n) * 1.5).astype(np.float32)
        x[[1, n // 3, n - 1]] = [np.inf, np.nan, -7e3]
        check(gpu_lib, x)
    announce("quantize bf16 n=4096*8192+8 (LDS-staged)")
    xb = rng.standard_normal(4096 * 8192 + 8).astype(np.float32)
    check(gpu_lib, wl.fp32_to_bf16_bits(xb), dtype="bf16")
    prev = gpu_lib.fp8_quantize_wait_ticks(0)
    try:
        announce("quantize fallback f32 n=4096*4096+4 (LDS-staged)")
        x = rng.standard_normal(4096 * 4096 + 4).astype(np.float32)
        check(gpu_lib, x)
    finally:
        gpu_lib.fp8_quantize_wait_ticks(prev)


def test_quantize_bf16_across_the_one_launch_limit(gpu_lib):
    """bf16 x holds 8 elements per 16-byte vector: 4096 x 8192 (64 MiB, 1024
    workgroups) is the largest bf16 tensor held in registers alone, 8 more
    elements take the LDS-staged instance; both match the oracle bit for
    bit."""
    rng = np.random.default_rng(34)
    n_one = 4096 * 8192
    for n in (n_one, n_one + 8):
        announce(f"quantize bf16 n={n}")
        x = rng.standard_normal(n).astype(np.float32)
        x[[5, n // 2]] = [np.nan, -np.inf]
        check(gpu_lib, wl.fp32_to_bf16_bits(x), dtype="bf16")


def test_quantize_fallback_reads_missing_ranges(gpu_lib):
    """With no wait for the other workgroups' maxima, every workgroup of the
    one-launch form reads the ranges whose maxima it has not seen yet: the
    slow path that keeps the result exact when workgroups are not resident
    together.  f32 and bf16, E4M3 and E5M2, with non-finite inputs."""
    rng = np.random.default_rng(32)
    prev = gpu_lib.fp8_quantize_wait_ticks(0)
    try:
        for shape, fmt in [((1024, 1024), "e4m3"), ((640, 2000), "e5m2")]:
            announce(f"quantize fallback f32 {shape} {fmt}")
            x = rng.standard_normal(shape).astype(np.float32)
            x[3, 7], x[-1, -1] = np.nan, -np.inf
            q, s, amax, bad = _quantize_dev(gpu_lib, dev(x), fmt=fmt)
            rq, rs, ramax, rbad = oracle.fp8_quantize(x, fmt=fmt)
            assert np.float32(host(s)[0]) == np.float32(rs)
            assert np.float32(host(amax)[0]) == np.float32(ramax) and int(host(bad)[0]) == rbad
            assert np.array_equal(host(q), rq)
        announce("quantize fallback bf16 (2048, 1536)")
        xb = wl.fp32_to_bf16_bits(rng.standard_normal((2048, 1536)).astype(np.float32))
        check(gpu_lib, xb, dtype="bf16")
    finally:
        gpu_lib.fp8_quantize_wait_ticks(prev)


def test_quantize_in_a_graph_matches_eager(gpu_lib):
    """Under graph capture the quantize takes its two-launch form (a replay
    would repeat the one-launch form's call tag): replays of the captured
    call, with eager calls and synchronisations between them, give the
    eager call's bits."""
    announce("quantize 4096 x 4096 f32: graph replays vs eager")
    rng = np.random.default_rng(33)
    x = dev((rng.standard_normal((4096, 4096)) * 2).astype(np.float32))
    eq, es, ea, eb = _quantize_dev(gpu_lib, x)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s, amax = scalar(0.0), scalar(0.0)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(gpu_lib.fp8_quantize_workspace_bytes(x.numel()), dtype=torch.uint8,
                     device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            gpu_lib.fp8_quantize(x, q, s, amax=amax, nonfinite=bad, ws=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        q.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, eq) and torch.equal(s, es) and torch.equal(amax, ea)
        assert torch.equal(bad, eb)
        _quantize_dev(gpu_lib, x)               # eager one-launch call between replays
        torch.cuda.synchronize()
