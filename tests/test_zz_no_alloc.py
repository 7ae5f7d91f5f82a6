"""fp8_quantize_noalloc (the entry point for callers that cannot allocate:
its amax partials live in the library's per-device scratch array) against
fp8_quantize with a caller workspace, through the C ABI: codes, scale, amax
and the non-finite count bit for bit, on two calls in a row whose second
input is smaller (the scratch keeps the first call's partials; the second
must not read them)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import announce, dev, host, scalar

pytestmark = pytest.mark.gpu


def run(fq, x, noalloc, fmt="e4m3", scale_in=None):
    q = torch.full(x.shape, 0x55, dtype=torch.uint8, device="cuda")
    s, amax = scalar(-1.0), scalar(-1.0)
    bad = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    si = None if scale_in is None else scalar(scale_in)
    if noalloc:
        fq.fp8_quantize_noalloc(x, q, s, scale_in=si, amax=amax, nonfinite=bad, fmt=fmt)
    else:
        fq.fp8_quantize(x, q, s, scale_in=si, amax=amax, nonfinite=bad, fmt=fmt)
    return host(q), host(s).view(np.uint32), host(amax).view(np.uint32), host(bad)


def same(a, b):
    return all(np.array_equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_noalloc_matches_workspace_call_twice(gpu_lib, fmt):
    rng = np.random.default_rng(5)
    # first call: large (1024 amax workgroups), with non-finite values and
    # an outlier; second call: much smaller, so a stale partial of the first
    # call (its maximum is larger) would change the scale
    big = (rng.standard_normal(4096 * 1024) * 3).astype(np.float32)
    big[123] = 9.0e3
    big[77] = np.nan
    big[4000] = -np.inf
    small = (rng.standard_normal(3000) * 0.5).astype(np.float32)
    for name, xn in (("4M elements", big), ("3000 elements", small)):
        announce(f"fp8_quantize_noalloc {fmt} {name}")
        x = dev(xn)
        a = run(gpu_lib, x, True, fmt)
        b = run(gpu_lib, x, False, fmt)
        assert same(a, b), name
    # bf16 input and a given scale, again large then small
    for n in (1 << 22, 1000):
        xb = dev((rng.standard_normal(n) * 2).astype(np.float32)).to(torch.bfloat16)
        assert same(run(gpu_lib, xb, True, fmt), run(gpu_lib, xb, False, fmt))
        assert same(run(gpu_lib, xb, True, fmt, 3.0), run(gpu_lib, xb, False, fmt, 3.0))


def test_noalloc_empty_and_graph_free_of_allocation(gpu_lib):
    """n = 0 writes s = 1 and amax = 0 as fp8_quantize does; and the call
    makes no allocation through torch's allocator (no workspace tensor)."""
    announce("fp8_quantize_noalloc n = 0 and allocator check")
    x0 = torch.zeros(0, dtype=torch.float32, device="cuda")
    assert same(run(gpu_lib, x0, True), run(gpu_lib, x0, False))
    x = dev(np.linspace(-5, 5, 1 << 20, dtype=np.float32))
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = scalar(0.0)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    gpu_lib.fp8_quantize_noalloc(x, q, s)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    assert float(host(s)[0]) == np.float32(448.0) / np.float32(5.0)
