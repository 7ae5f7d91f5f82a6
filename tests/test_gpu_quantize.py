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
