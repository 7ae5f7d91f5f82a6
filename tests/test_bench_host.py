"""Host-side parts of bench.py (no GPU): the one-GPU guard, the traffic
record's source check, and the argument surface."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_measured_sources(monkeypatch):
    # the committed summary records the digest of the GEMM sources it was
    # measured on; any other digest (changed sources) gives no traffic figure
    # and on the forward route it was measured on
    measured = [bench.gemm_traffic_bytes(f) for f in (False, True)]
    assert None in measured                               # one route only
    assert all(v is None or v > 96 * 2**20 for v in measured)   # >= the algorithmic bytes
    monkeypatch.setattr(bench, "gemm_sources_digest", lambda: "0" * 64)
    assert bench.gemm_traffic_bytes(False) is None and bench.gemm_traffic_bytes(True) is None


@pytest.mark.parametrize("argv", [["--workload", "mlp7b"], ["--workload", "rank-sweep"],
                                  ["--fp4-gemm"], ["--merge-every", "4"], ["--topk-rank", "16"],
                                  ["--workload", "rank-sweep", "--ranks", "8192"]])
def test_options_parse(monkeypatch, argv):
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    a = bench.parse()
    assert a.gpus == 1 and a.steps > 0 and a.warmup >= 0


def test_cpu_baseline_reports_the_oracle_step():
    """cpu_baseline times the oracle as it is on a token sample of the
    workload (one repetition here) and reports what it ran."""
    import workloads as wl
    spec = wl.WORKLOADS[1].linears[0]                 # the 512 x 512 single linear
    d0 = wl.make_linear(1, 0, spec, step=0)
    r = bench.cpu_baseline(spec, d0, 64, min_seconds=0.0, one_thread_tokens=32,
                           one_thread_seconds=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] >= 1 and r["tokens_per_s"] > 0
    assert "first 64 of 256 tokens" in r["sample"] and "1 repetition," in r["sample"]
    one = r["one_thread"]
    assert one["cores"] == 1 and one["value"] > 0 and "first 32 tokens" in one["sample"]
    import oracle
    assert oracle.num_threads() == r["cores"] or oracle.num_threads() >= 1   # restored


def test_timing_events_are_not_destroyed_by_finalizers():
    """HIP events are destroyed explicitly (TimingEvent.destroy_all after a
    synchronize), never from a finalizer that could run after the runtime."""
    assert not hasattr(bench.TimingEvent, "__del__")
    assert callable(bench.TimingEvent.destroy_all)


def test_rank_subset_of_the_sweep():
    import workloads as wl
    assert bench.sweep_ranks("", wl.RANK_SWEEP) == tuple(wl.RANK_SWEEP)
    # the sweep's order, whatever the order given
    assert bench.sweep_ranks("8192,512", wl.RANK_SWEEP) == (512, 8192)
    for bad in ("7", "64,100", ","):
        with pytest.raises(SystemExit):
            bench.sweep_ranks(bad, wl.RANK_SWEEP)
