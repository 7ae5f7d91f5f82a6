"""Benchmark of the melded FP8 LoRA linear training step on one MI355X.

Workload (the 7B attention projection): W 4096 x 4096 in E4M3, 4096 tokens
(batch 4 x sequence 1024) of N(0,1) activations with 1% outlier channels
scaled x20, dY ~ N(0, 1e-3), rank 64, SGD lr 1e-3, row-wise proxy update
every step.  One step = fp8_quantize(X) + melded_linear_fwd +
fp8_quantize(dY) + melded_linear_bwd (dX, dA, dB) + adapter_step (SGD, or
adapter_step_adamw with --optimizer adamw) +
rowwise_proxy_update, launched eagerly on one HIP stream, inputs resident in
HBM.

Prints ONE JSON line.  `value` is whole-step TFLOP/s over the algorithmic
flops of a step (forward and dX FP8 GEMMs, the four rank-r adapter
contractions and the rank-r row delta); tokens/s is reported beside it.
`roofline` describes the dominant kernel (the forward FP8 GEMM), timed with
HIP events on the stream it runs on.  `cpu_baseline` times the CPU oracle on
a token sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "melded FP8 LoRA linear fwd+bwd TFLOP/s and tokens/s; % FP8 MFMA / HBM peak"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
FP32_PEAK_TFLOPS = 157.3      # MI355X dense fp32 (matrix and vector)


class TimingEvent:
    """A HIP event used only for timing, created with
    hipEventDisableSystemFence: recording it does not write back and
    invalidate the caches.  An ordinary timing event does, and in a kernel
    trace of the step each such record left about 6 us of idle GPU after it
    and lengthened the kernel that followed.  The timestamps are the same GPU
    clock; read elapsed times only after a device synchronize.

    Lifetime: every event is kept in a class-wide list and destroyed by
    destroy_all() before main() returns, after a device synchronize.  No HIP
    call is made from a finalizer: at interpreter exit the HIP runtime (and a
    profiler's interception of it) may already be torn down."""

    _hip = None
    _live = []
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            # the HIP runtime torch has loaded (the same shared object)
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._c = ctypes
        self.ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.ev),
                                               ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        TimingEvent._live.append(self)

    def record(self, stream):
        rc = self._hip.hipEventRecord(self.ev, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end`."""
        ms = self._c.c_float()
        rc = self._hip.hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self):
        if self.ev:
            self._hip.hipEventDestroy(self.ev)
            self.ev = self._c.c_void_p()

    @classmethod
    def destroy_all(cls):
        """Destroy every event made so far (call after a device synchronize)."""
        for e in cls._live:
            e.destroy()
        cls._live.clear()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--chunk", type=int, default=10,
                    help="timed steps per chunk: the median over the chunks' per-step "
                         "times is reported beside the mean")
    ap.add_argument("--batches", type=int, default=4, help="distinct (X, dY) batches cycled")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="token sample for the CPU-oracle baseline (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--adapter", choices=["trained", "frozen-fp8"], default="trained",
                    help="A trained in fp32 (dA computed), or the pages' training setup: A "
                         "frozen in FP8, X~A~^T formed in the forward, no dA")
    ap.add_argument("--topk-rank", type=int, default=0,
                    help="merge only the top-k rank components of the proxy (0: all r)")
    ap.add_argument("--grad-format", choices=["e4m3", "e5m2"], default="e4m3",
                    help="FP8 format of the upstream gradient dY")
    ap.add_argument("--merge-every", type=int, default=1,
                    help="run the row-wise proxy update on every N-th step (B accumulates "
                         "the adapter updates in between)")
    ap.add_argument("--optimizer", choices=["sgd", "adamw"], default="sgd",
                    help="adapter optimizer: SGD lr 1e-3 (the workload's) or 32-bit AdamW "
                         "(the pages' training runs)")
    ap.add_argument("--fp4-gemm", action="store_true",
                    help="also time the forward product with FP4 E2M1 operands (X and W cast "
                         "by fp4_quantize) against the FP8 one, alternating launches")
    ap.add_argument("--workload", choices=["attn7b", "mlp7b", "layer13b", "rank-sweep"],
                    default="attn7b",
                    help="attn7b: the 7B attention projection (the headline line); mlp7b: the "
                         "three 7B MLP linears, 8192 bf16 tokens; layer13b: the seven linears of "
                         "a 13B decoder layer, 4096 tokens; rank-sweep: 4096 x 4096, 8192 "
                         "tokens, r in 8 .. 8192 (fwd + bwd time and step time per rank)")
    ap.add_argument("--compare-paths", action="store_true",
                    help="with --workload rank-sweep: also time the separate-path FP8 LoRA "
                         "layer and the bf16 LoRA layer at every rank (fwd + bwd), and the FP8 "
                         "backbone alone")
    ap.add_argument("--ranks", type=str, default="",
                    help="with --workload rank-sweep: a comma-separated subset of the sweep's "
                         "ranks (default all); without 64 the line's value is the first "
                         "rank's point")
    ap.add_argument("--gemm-event-every", type=int, default=10,
                    help="bracket the forward GEMM with timing events on every N-th timed "
                         "step (1 = every step)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the timed steps "
                         "(calibrates the HBM byte counters of a profiler run)")
    return ap.parse_args()


def main():
    args = parse()
    try:
        run(args)
    finally:
        # explicit teardown while the HIP runtime is alive: drain the GPU,
        # then destroy the timing events (nothing is left to finalizers)
        if "torch" in sys.modules:
            import torch
            if torch.cuda.is_initialized():
                torch.cuda.synchronize()
                TimingEvent.destroy_all()


def run(args):
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the per-GPU shard of the step is what one GPU runs); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_quantized_lora_amd as fq
    import workloads as wl

    fq.load()
    torch.cuda.set_device(0)
    if args.workload != "attn7b":
        if args.adapter != "trained" or args.topk_rank or args.grad_format != "e4m3" or \
                args.merge_every != 1 or args.optimizer != "sgd" or args.fp4_gemm:
            sys.exit("--workload other than attn7b runs the default step only")
        out = (rank_sweep(args, torch, fq, wl) if args.workload == "rank-sweep"
               else layer_workload(args, torch, fq, wl))
        print(json.dumps(out), flush=True)
        return
    cfg = wl.WORKLOADS[2]
    spec = cfg.linears[0]
    T, d_in, d_out, r = spec.tokens, spec.d_in, spec.d_out, spec.rank

    d0 = wl.make_linear(2, 0, spec, step=0)
    frozen = args.adapter == "frozen-fp8"
    m = fq.MeldedLinear(d_out, d_in, r, T, optimizer=args.optimizer, fp8_a=frozen,
                        g_fmt=args.grad_format, topk_rank=args.topk_rank,
                        merge_every=max(1, args.merge_every))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    m.init_state(t(d0["W"]), t(d0["A"]), t(d0["B"]))
    batches = []
    for b in range(max(1, args.batches)):
        d = d0 if b == 0 else wl.step_activations(2, 0, spec, b)
        batches.append((t(d["X"]), t(d["dY"])))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    names = ["quantize_x", "fwd_gemm", "quantize_dy", "bwd", "adapter_step", "proxy_update"]

    if args.merge_every < 1:
        sys.exit("--merge-every must be >= 1")
    if args.gemm_event_every < 1:
        sys.exit("--gemm-event-every must be >= 1")

    def merges(i):
        """whether step i (0-based) ends with the proxy update"""
        return (i + 1) % args.merge_every == 0

    def calls(i):
        """The step's six boundary calls for batch i, in order (the last one a
        no-op on steps without a merge)."""
        X, dY = batches[i % len(batches)]
        return [
            lambda: fq.fp8_quantize(X, m.xq, m.s_x, ws=m.ws_q, stream=stream),
            lambda: m.forward_product(stream),
            lambda: fq.fp8_quantize(dY, m.gq, m.s_g, ws=m.ws_q, stream=stream,
                                    fmt=args.grad_format),
            lambda: m.backward_product(stream),
            lambda: m.adapter_update(spec.lr, stream=stream),
            (lambda: m.merge(spec.tau, spec.k_max, stream=stream)) if merges(i)
            else (lambda: None),
        ]

    for i in range(args.warmup):
        for c in calls(i):
            c()
    torch.cuda.synchronize()

    # Per-call durations (reported beside the result, not part of the timed
    # region): HIP events between the calls of a few eager steps.
    n_pc = max(3, min(args.steps, 10), args.merge_every)
    pc = [[TimingEvent() for _ in range(len(names) + 1)]
          for _ in range(n_pc)]
    for i in range(n_pc):
        for k, c in enumerate(calls(args.warmup + i)):
            pc[i][k].record(stream)
            c()
        pc[i][len(names)].record(stream)
    torch.cuda.synchronize()
    per_call_us = {n: sum(pc[i][k].elapsed_time(pc[i][k + 1]) for i in range(n_pc)) * 1e3 / n_pc
                   for k, n in enumerate(names)}
    # the proxy update's own duration: averaged over the steps that ran it
    n_merge = sum(merges(args.warmup + i) for i in range(n_pc))
    per_call_us["proxy_update"] = sum(
        pc[i][5].elapsed_time(pc[i][6]) for i in range(n_pc) if merges(args.warmup + i)
    ) * 1e3 / max(1, n_merge)

    # Copy-kernel reference (not part of the timed region): a 256 MiB device
    # copy whose source was evicted from the 256 MB last-level cache by a
    # 1 GiB write, timed with HIP events; the bandwidth kernels are also
    # reported as a fraction of this measured rate.
    copy_gbs = copy_reference_gbs(torch, stream)

    # A plain device copy of known size, for scaling the HBM byte counters of
    # a profiler run (not part of the timed region).
    # The source is written, then 1 GiB of other data is written so that the
    # copy reads its source from HBM rather than from the 256 MB last-level
    # cache.
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18                       # float32 elements
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        evict = torch.empty(1 << 28, device="cuda")
        evict.fill_(2.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, evict

    # Timed region: K steps, launched eagerly on one stream (back-to-back
    # launches keep the GPU busy: a captured-graph replay of the step measured
    # no faster).  The forward FP8 GEMM, the dominant kernel, is bracketed by
    # HIP timing events (without the cache-flushing fence) on the stream it
    # runs on, so its launch duration is measured in the same region: on
    # every tenth step (and the first), since each event record still
    # leaves a few microseconds of idle GPU on the stream (with a pair on
    # every step the step measured ~6 us longer).
    sampled = [i for i in range(args.steps) if i % args.gemm_event_every == 0]
    g_ev = {i: (TimingEvent(), TimingEvent()) for i in sampled}
    # chunk boundaries: an event before step 0 and after every `chunk` steps
    # (one record per chunk costs the stream a few microseconds once per
    # chunk), so the median step time over the chunks is measured in the same
    # region as the total
    chunk = max(1, args.chunk)
    bounds = sorted(set(list(range(0, args.steps, chunk)) + [args.steps]))
    c_ev = {b: TimingEvent() for b in bounds}
    torch.cuda.synchronize()
    for i in range(args.steps):
        if i in c_ev:
            c_ev[i].record(stream)
        for k, c in enumerate(calls(args.warmup + n_pc + i)):
            if k == 1 and i in g_ev:
                g_ev[i][0].record(stream)
                c()
                g_ev[i][1].record(stream)
            else:
                c()
    c_ev[args.steps].record(stream)
    torch.cuda.synchronize()
    ms_per_step = c_ev[0].elapsed_time(c_ev[args.steps]) / args.steps
    chunk_ms = sorted(c_ev[a].elapsed_time(c_ev[b]) / (b - a) for a, b in zip(bounds, bounds[1:]))
    ms_median = chunk_ms[len(chunk_ms) // 2] if len(chunk_ms) % 2 else \
        0.5 * (chunk_ms[len(chunk_ms) // 2 - 1] + chunk_ms[len(chunk_ms) // 2])
    gemm_timed_us = sum(a.elapsed_time(b) for a, b in g_ev.values()) * 1e3 / len(g_ev)
    n_sel = int(m.n_sel.cpu()[0])

    # the row delta B.A (rank r, or the top-k components) on merge steps only
    n_merge_timed = sum(merges(args.warmup + n_pc + i) for i in range(args.steps))
    chain = 2 * d_out * d_in * (args.topk_rank or r)
    flops = (wl.step_flops(T, d_in, d_out, r, frozen_a=frozen) - 2 * d_out * d_in * r
             + chain * n_merge_timed / args.steps)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = T / (ms_per_step * 1e-3)
    # the forward call's algorithmic flops: the backbone product, plus the
    # rank-r product X^ A^T (X~ A~^T with A frozen) where the call forms it
    # (counted once, at rank r, though the fused route carries A as three
    # E4M3 pieces under block scales)
    gemm_flops = 2 * T * d_in * d_out + (2 * T * d_in * r if frozen or m.use_xa else 0)
    gemm_us = gemm_timed_us
    gemm_tflops = gemm_flops / (gemm_us * 1e-6) / 1e12
    quant_bytes = T * d_in * 5 + 4                  # fp32 in, E4M3 out, the scale
    quant_gbs = quant_bytes / (per_call_us["quantize_x"] * 1e-6) / 1e9
    # proxy update: read the codes, A and B; write the selected rows' codes,
    # zero their B rows, write the indices
    proxy_bytes = d_out * d_in + 4 * r * (d_in + d_out) + n_sel * (d_in + 4 * r + 4)
    proxy_gbs = proxy_bytes / (per_call_us["proxy_update"] * 1e-6) / 1e9
    # the proxy update's exact chain runs on the fp32 matrix cores: 2 r flops
    # per backbone element (r = the merged components)
    proxy_tflops = chain / (per_call_us["proxy_update"] * 1e-6) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "median_over": f"{len(chunk_ms)} chunks of {chunk} steps",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "7B attention projection: W 4096x4096 E4M3, 4096 tokens "
                               "(4 x 1024), 1% outlier channels x20, rank 64, "
                               + ("SGD" if args.optimizer == "sgd" else "32-bit AdamW")
                               + " lr 1e-3, proxy update every "
                               + ("step" if args.merge_every == 1 else f"{args.merge_every} steps")
                               + (", A frozen in FP8 (X~A~^T formed in the forward, no dA)"
                                  if frozen else "")
                               + (", dY in E5M2" if args.grad_format == "e5m2" else "")
                               + (f", proxy merges the top {args.topk_rank} rank components"
                                  if args.topk_rank else ""),
                   "tokens": T, "d_in": d_in, "d_out": d_out, "rank": r,
                   "optimizer": args.optimizer, "adapter": args.adapter,
                   "merge_every": args.merge_every, "grad_format": args.grad_format,
                   "topk_rank": args.topk_rank,
                   "parallelism": "single GPU"},
        "tokens_per_s": round(tokens_per_s, 1),
        "roofline": {"kernel": ("melded_linear_fwd_frozen_a call (FP8 GEMM 4096 x 4096 x 4096 "
                                "+ X~A~^T)" if frozen else
                                "melded_linear_fwd_xa_pieces call (one FP8 GEMM 4096 x 4096 x "
                                "4096 forming X^A^T in the same tiles from A's block-scaled E4M3 "
                                "pieces, which the SGD step leaves)"
                                if m.keep_pieces else
                                "melded_linear_fwd_xa call (A as block-scaled E4M3 pieces, then "
                                "one FP8 GEMM 4096 x 4096 x 4096 forming X^A^T in the same tiles)"
                                if m.use_xa else
                                "melded_linear_fwd FP8 GEMM (4096 x 4096 x 4096)"),
                     "bound": "mfma", "achieved": round(gemm_tflops, 1),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": None if frozen else gemm_traffic_bytes(m.use_xa)},
        "per_call_us": {k: round(v, 2) for k, v in per_call_us.items()},
        "launch": "eager launches on one HIP stream",
        "fwd_gemm_us_timed": round(gemm_timed_us, 2),
        "fwd_gemm_timed_launches": len(g_ev),
        "quantize_x_GBps": round(quant_gbs, 1),
        "quantize_x_hbm_frac": round(quant_gbs / HBM_PEAK_GBS, 4),
        "copy_reference_GBps": round(copy_gbs, 1),
        "quantize_x_frac_of_copy": round(quant_gbs / copy_gbs, 4),
        "proxy_update_GBps": round(proxy_gbs, 1),
        "proxy_update_hbm_frac": round(proxy_gbs / HBM_PEAK_GBS, 4),
        "proxy_update_frac_of_copy": round(proxy_gbs / copy_gbs, 4),
        "proxy_update_chain_TFLOPs": round(proxy_tflops, 1),
        "proxy_update_fp32_mfma_frac": round(proxy_tflops / FP32_PEAK_TFLOPS, 4),
        "selected_rows_last_step": n_sel,
    }

    if args.fp4_gemm:
        out["fp4_forward"] = fp4_forward(torch, fq, batches[0][0], t(d0["W"]), m, stream)

    if not args.no_cpu_baseline and args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(spec, d0, args.cpu_tokens, args.optimizer, frozen,
                                           args.grad_format)
    print(json.dumps(out), flush=True)


def _upload(torch, np, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _linear_state(torch, np, fq, wl, cfg_id, li, spec, rank=None):
    """A MeldedLinear initialised from the workload's seeded W, A, B, with the
    step-0 X (bf16 where the workload passes bf16) and dY resident."""
    r = spec.rank if rank is None else rank
    d = wl.make_linear(cfg_id, li, spec, step=0, rank=r)
    x_dtype = torch.bfloat16 if spec.x_bf16 else torch.float32
    m = fq.MeldedLinear(spec.d_out, spec.d_in, r, spec.tokens, x_dtype=x_dtype)
    m.init_state(_upload(torch, np, d["W"]), _upload(torch, np, d["A"]),
                 _upload(torch, np, d["B"]))
    if spec.x_bf16:
        X = _upload(torch, np, d["X_bf16"].view(np.int16)).view(torch.bfloat16)
    else:
        X = _upload(torch, np, d["X"])
    dY = _upload(torch, np, d["dY"])
    return m, X, dY, d


def _step_calls(fq, m, X, dY, spec, stream):
    """The six boundary calls of one melded-linear step."""
    return [
        lambda: fq.fp8_quantize(X, m.xq, m.s_x, ws=m.ws_q, stream=stream),
        lambda: m.forward_product(stream),
        lambda: fq.fp8_quantize(dY, m.gq, m.s_g, ws=m.ws_q, stream=stream),
        lambda: m.backward_product(stream),
        lambda: m.adapter_update(spec.lr, stream=stream),
        lambda: m.merge(spec.tau, spec.k_max, stream=stream),
    ]


def _timed(torch, steps, warmup, run_step, stream, gemm=True):
    """Warm-up, then `steps` steps between two timing events.  `run_step(i,
    ev)` runs step i; with `gemm`, ev is a pair of timing events the step
    records around its dominant GEMM (None during warm-up).  Returns (ms per
    step, GEMM us per launch or None)."""
    for i in range(warmup):
        run_step(i, None)
    torch.cuda.synchronize()
    g_ev = [(TimingEvent(), TimingEvent()) if gemm else None for _ in range(steps)]
    start, stop = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        run_step(warmup + i, g_ev[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    gemm_us = sum(a.elapsed_time(b) for a, b in g_ev) * 1e3 / steps if gemm else None
    return ms, gemm_us


def _run_calls(calls, ev, stream, gemm_index=1):
    for k, c in enumerate(calls):
        if ev is not None and k == gemm_index:
            ev[0].record(stream)
            c()
            ev[1].record(stream)
        else:
            c()


def layer_workload(args, torch, fq, wl):
    """The 7B MLP (three linears, 8192 bf16 tokens) or the 13B decoder layer
    (seven linears, 4096 tokens): one step runs every linear's step in turn,
    each with its own seeded state, X and dY.  The dominant kernel is the
    forward GEMM of the first linear (the largest shape of both layers)."""
    import numpy as np
    cfg_id = 3 if args.workload == "mlp7b" else 4
    cfg = wl.WORKLOADS[cfg_id]
    stream = torch.cuda.current_stream()
    layers = []
    for li, spec in enumerate(cfg.linears):
        m, X, dY, d = _linear_state(torch, np, fq, wl, cfg_id, li, spec)
        layers.append((m, X, dY, spec))
        if li == 0:
            d0 = d
        del d
    torch.cuda.synchronize()

    def run_step(i, ev):
        for li, (m, X, dY, spec) in enumerate(layers):
            _run_calls(_step_calls(fq, m, X, dY, spec, stream), ev if li == 0 else None, stream)

    ms, gemm_us = _timed(torch, args.steps, args.warmup, run_step, stream)
    flops = sum(wl.step_flops(sp.tokens, sp.d_in, sp.d_out, sp.rank) for _, _, _, sp in layers)
    s0 = layers[0][3]
    m0 = layers[0][0]
    T = s0.tokens
    # the timed forward call: the backbone product, plus X^ A^T where the
    # call forms it in the same tiles (counted once, at rank r)
    gemm_flops = 2 * T * s0.d_in * s0.d_out + (2 * T * s0.d_in * s0.rank if m0.use_xa else 0)
    gemm_tf = gemm_flops / (gemm_us * 1e-6) / 1e12
    shapes = ", ".join(f"{sp.name} {sp.d_out}x{sp.d_in}" for _, _, _, sp in layers)
    out = {
        "metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": ("7B MLP" if cfg_id == 3 else "13B decoder layer")
                   + f" ({shapes}; W E4M3), {T} tokens"
                   + (" of bf16 activations" if s0.x_bf16 else "")
                   + ", rank 64, SGD lr 1e-3, proxy update every step; one step runs every "
                     "linear once; the same X and dY every step",
                   "tokens": T, "linears": len(layers), "rank": s0.rank,
                   "parallelism": "single GPU"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"kernel": (f"melded_linear_fwd_xa_pieces call ({s0.name}: one FP8 GEMM {T} "
                                f"x {s0.d_out} x {s0.d_in} forming X^A^T in the same tiles from "
                                f"A's pieces, which the SGD step leaves)" if m0.keep_pieces else
                                f"melded_linear_fwd_xa call ({s0.name}: A as block-scaled E4M3 "
                                f"pieces, then one FP8 GEMM {T} x {s0.d_out} x {s0.d_in} forming "
                                f"X^A^T in the same tiles)" if m0.use_xa else
                                f"melded_linear_fwd FP8 GEMM ({T} x {s0.d_out} x {s0.d_in}, "
                                f"{s0.name})"),
                     "bound": "mfma", "achieved": round(gemm_tf, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tf / FP8_PEAK_TFLOPS, 4),
                     "traffic": None},
        "launch": "eager launches on one HIP stream",
    }
    if not args.no_cpu_baseline and args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(s0, d0, min(args.cpu_tokens, 512),
                                           x_note=" (bf16 activations widened exactly)"
                                           if s0.x_bf16 else "")
    return out


def compare_paths(torch, fq, m, X, dY, args, stream, melded_ms):
    """fwd+bwd times of the FP8 backbone alone, of the separate-path FP8 LoRA
    layer and of the bf16 LoRA layer, on the melded layer m's inputs."""
    T, d_in, d_out, r = m.T, m.d_in, m.d_out, m.r
    dev = m.wq.device
    u8, f32 = torch.uint8, torch.float32
    e_in = torch.empty((0, d_in), dtype=f32, device=dev)
    e_out = torch.empty((d_out, 0), dtype=f32, device=dev)
    qx = lambda: fq.fp8_quantize(X, m.xq, m.s_x, ws=m.ws_q, stream=stream)  # noqa: E731
    qg = lambda: fq.fp8_quantize(dY, m.gq, m.s_g, ws=m.ws_q, stream=stream)  # noqa: E731
    fwd = lambda: fq.melded_linear_fwd(m.xq, m.s_x, m.wq, m.s_w, m.y, stream=stream)  # noqa: E731
    base = [qx, fwd, qg, lambda: fq.melded_linear_bwd(m.gq, m.s_g, m.xq, m.s_x, m.wq, m.s_w,
                                                       e_in, e_out, m.dx, e_in, e_out,
                                                       ws=m.ws_bwd, stream=stream)]
    sv = torch.empty(fq.lora_separate_fp8_saved_bytes(T, d_in, d_out, r), dtype=u8, device=dev)
    wsv = torch.empty(fq.lora_separate_fp8_workspace_bytes(T, d_in, d_out, r), dtype=u8,
                      device=dev)
    sep = [qx, lambda: fq.lora_separate_fp8_fwd(m.xq, m.s_x, m.wq, m.s_w, m.A, m.B, m.y, sv,
                                                ws=wsv, stream=stream),
           qg, lambda: fq.lora_separate_fp8_bwd(m.gq, m.s_g, m.xq, m.s_x, m.wq, m.s_w, sv, r,
                                                m.dx, m.dA, m.dB, ws=wsv, stream=stream)]
    Xf = X.float() if X.dtype != torch.float32 else X
    sb = torch.empty(fq.lora_bf16_saved_bytes(T, d_in, d_out, r), dtype=u8, device=dev)
    wsb = torch.empty(fq.lora_bf16_workspace_bytes(T, d_in, d_out, r), dtype=u8, device=dev)
    bf = [qx, lambda: fq.lora_bf16_fwd(Xf, m.xq, m.s_x, m.wq, m.s_w, m.A, m.B, m.y, sb, ws=wsb,
                                       stream=stream),
          qg, lambda: fq.lora_bf16_bwd(dY, m.gq, m.s_g, Xf, m.wq, m.s_w, m.A, m.B, sb, m.dx,
                                       m.dA, m.dB, ws=wsb, stream=stream)]
    res = {}
    for name, cl in (("backbone", base), ("separate_fp8", sep), ("bf16", bf)):
        ms, _ = _timed(torch, args.steps, args.warmup,
                       lambda i, ev: _run_calls(cl, None, stream), stream, gemm=False)
        res[name] = ms
    del sv, wsv, sb, wsb
    return {"backbone_fwd_bwd_ms": round(res["backbone"], 4),
            "separate_fp8_fwd_bwd_ms": round(res["separate_fp8"], 4),
            "bf16_fwd_bwd_ms": round(res["bf16"], 4),
            "melded_adapter_ms": round(melded_ms - res["backbone"], 4),
            "separate_fp8_adapter_ms": round(res["separate_fp8"] - res["backbone"], 4),
            "bf16_adapter_ms": round(res["bf16"] - res["backbone"], 4),
            "melded_over_separate_speedup": round(res["separate_fp8"] / melded_ms, 3)}


def sweep_ranks(spec: str, allowed):
    """The ranks named by --ranks (a comma-separated subset of `allowed`, in
    the sweep's order), or all of them."""
    if not spec:
        return tuple(allowed)
    want = {int(t) for t in spec.split(",") if t.strip()}
    bad = sorted(want - set(allowed))
    if bad or not want:
        raise SystemExit(f"--ranks: {bad or spec!r} not in the sweep's ranks {tuple(allowed)}")
    return tuple(r for r in allowed if r in want)


def rank_sweep(args, torch, fq, wl):
    """W 4096 x 4096, 8192 tokens, r in 8, 64, 512, 2048, 8192: per rank the
    forward + backward time (quantize X, forward, quantize dY, backward) and
    the whole step's (plus SGD and the proxy update), each timed over its own
    eager steps.  The line's value is the step TFLOP/s at r = 64."""
    import numpy as np
    cfg = wl.WORKLOADS[5]
    spec0 = cfg.linears[0]
    stream = torch.cuda.current_stream()
    points = []
    line = None
    ranks = sweep_ranks(args.ranks, wl.RANK_SWEEP)
    line_rank = 64 if 64 in ranks else ranks[0]
    for r in ranks:
        m, X, dY, d = _linear_state(torch, np, fq, wl, 5, 0, spec0, rank=r)
        spec = dataclasses.replace(spec0, rank=r)
        calls = _step_calls(fq, m, X, dY, spec, stream)
        fb_ms, _ = _timed(torch, args.steps, args.warmup,
                          lambda i, ev: _run_calls(calls[:4], None, stream), stream, gemm=False)
        ms, gemm_us = _timed(torch, args.steps, args.warmup,
                             lambda i, ev: _run_calls(calls, ev, stream), stream)
        T = spec.tokens
        fb_flops = 4 * T * spec.d_in * spec.d_out + 4 * T * r * (spec.d_in + spec.d_out)
        flops = wl.step_flops(T, spec.d_in, spec.d_out, r)
        n_sel = int(m.n_sel.cpu()[0])
        point = {"rank": r, "fwd_bwd_ms": round(fb_ms, 4), "step_ms": round(ms, 4),
                 "fwd_bwd_TFLOPs": round(fb_flops / (fb_ms * 1e-3) / 1e12, 1),
                 "step_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                 "fwd_gemm_us": round(gemm_us, 2),
                 "selected_rows_last_step": n_sel}
        if args.compare_paths:
            point.update(compare_paths(torch, fq, m, X, dY, args, stream, fb_ms))
        points.append(point)
        if r == line_rank:
            line = (ms, gemm_us, d, spec, m.use_xa)
        del m, X, dY, d, calls
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.compare_paths:
        # the smallest rank from which the FP8 branch (separate path) costs
        # less than the bf16 one
        tp = [q["rank"] for q in points if q["separate_fp8_adapter_ms"] < q["bf16_adapter_ms"]]
        turning = tp[0] if tp else None
    ms, gemm_us, d64, spec64, xa64 = line
    T = spec64.tokens
    # the timed forward call: the backbone product, plus X^ A^T where the call
    # forms it in the same tiles (counted once, at rank r)
    gemm_flops = 2 * T * spec64.d_in * (spec64.d_out + (line_rank if xa64 else 0))
    gemm_tf = gemm_flops / (gemm_us * 1e-6) / 1e12
    out = {
        "metric": METRIC,
        "value": round(wl.step_flops(T, spec64.d_in, spec64.d_out, line_rank) / (ms * 1e-3) / 1e12,
                       2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": "rank sweep: W 4096x4096 E4M3, 8192 tokens, A std 1/sqrt(r), "
                               "B std 1e-3, SGD lr 1e-3, proxy update every step; the "
                               f"line's value and ms_per_step are the r = {line_rank} point",
                   "tokens": T, "d_in": spec64.d_in, "d_out": spec64.d_out,
                   "ranks": list(ranks), "parallelism": "single GPU"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"kernel": f"forward call FP8 GEMM ({T} x 4096 x 4096"
                               f"{', forming X^A^T' if xa64 else ''}), r = {line_rank} point",
                     "bound": "mfma", "achieved": round(gemm_tf, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tf / FP8_PEAK_TFLOPS, 4),
                     "traffic": None},
        "sweep": points,
        "launch": "eager launches on one HIP stream",
    }
    if args.compare_paths:
        out["fp8_vs_bf16_adapter_turning_rank"] = turning
        out["compare_paths_note"] = (
            "fwd+bwd of one layer (both quantizes, forward, backward) on the same inputs: "
            "melded (the adapter inside the FP8 backbone), separate-path FP8 LoRA (adapter "
            "branch with its own E4M3 quantizes, FP8 matrix cores) and bf16 LoRA (adapter "
            "branch in bfloat16); *_adapter_ms = the path's time minus the FP8 backbone alone "
            "(quantizes, forward GEMM, dX)")
    if not args.no_cpu_baseline and args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(spec64, d64, min(args.cpu_tokens, 1024))
    return out


FP4_PEAK_TFLOPS = 10100.0     # MI355X dense FP4 matrix peak


def fp4_forward(torch, fq, X, W, m, stream, reps=20):
    """The forward product with FP4 E2M1 operands (the pages' Table R3
    estimates an FP4 speed-up from the FP4/FP8 matrix throughput ratio; this
    measures it): X and W cast by fp4_quantize, melded_linear_fwd_fp4 and the
    FP8 melded_linear_fwd launched alternately, each between HIP events on
    the bench stream."""
    T, d_in = X.shape
    d_out = W.shape[0]
    xq4 = torch.empty((T, d_in // 2), dtype=torch.uint8, device="cuda")
    wq4 = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device="cuda")
    sx4 = torch.zeros(1, device="cuda")
    sw4 = torch.zeros(1, device="cuda")
    y4 = torch.empty((T, d_out), device="cuda")
    fq.fp4_quantize(X, xq4, sx4, stream=stream)
    fq.fp4_quantize(W, wq4, sw4, stream=stream)
    f4 = lambda: fq.melded_linear_fwd_fp4(xq4, sx4, wq4, sw4, y4, stream=stream)  # noqa: E731
    f8 = lambda: fq.melded_linear_fwd(m.xq, m.s_x, m.wq, m.s_w, m.y, stream=stream)  # noqa: E731
    for _ in range(3):
        f4()
        f8()
    ev = [[TimingEvent() for _ in range(4)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        f4()
        e[1].record(stream)
        e[2].record(stream)
        f8()
        e[3].record(stream)
    torch.cuda.synchronize()
    us4 = sum(e[0].elapsed_time(e[1]) for e in ev) * 1e3 / reps
    us8 = sum(e[2].elapsed_time(e[3]) for e in ev) * 1e3 / reps
    flops = 2.0 * T * d_in * d_out
    tf4 = flops / (us4 * 1e-6) / 1e12
    return {"gemm_us": round(us4, 2), "achieved_TFLOPs": round(tf4, 1),
            "peak_TFLOPs": FP4_PEAK_TFLOPS, "frac": round(tf4 / FP4_PEAK_TFLOPS, 4),
            "fp8_gemm_us_same_run": round(us8, 2),
            "fp4_over_fp8_speedup": round(us8 / us4, 3),
            "shape": f"{T} x {d_out} x {d_in}, operands cast to E2M1 by fp4_quantize"}


def copy_reference_gbs(torch, stream, mib=256, reps=5):
    """Bytes read + written per second by a plain device-to-device copy of
    `mib` MiB whose source is first pushed out of the last-level cache (median
    of `reps`)."""
    n = mib << 18
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    evict = torch.empty(1 << 28, device="cuda")
    times = []
    with torch.cuda.stream(stream):
        for _ in range(reps):
            evict.fill_(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
    del src, dst, evict
    times.sort()
    return 2 * n * 4 / times[len(times) // 2] / 1e9


GEMM_SOURCES = ("fp8_quantized_lora_amd/csrc/gemm_fp8_kernel.hpp",
                "fp8_quantized_lora_amd/csrc/gemm_fp8.hip",
                "fp8_quantized_lora_amd/csrc/common.hpp")
TRAFFIC_SUMMARY = "profiles/gemm_fp8_nt_dma_4096x4096x4096_hbm_traffic.md"


def gemm_sources_digest():
    """sha256 over the GEMM sources with comments and blank space removed, so
    that only code changes invalidate a traffic measurement."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def gemm_traffic_bytes(fused_xa):
    """HBM bytes per launch of the 4096^3 FP8 GEMM from the committed
    FETCH_SIZE / WRITE_SIZE counter summary, or None when that summary is
    missing, was taken on other kernel sources than the ones built here, or
    on the other forward route (`fused_xa`: X^ A^T formed in the GEMM's
    tiles)."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                vals[k.strip("`")] = v.strip().strip("`")
    if vals.get("sources_sha256") != gemm_sources_digest():
        return None
    if vals.get("forward_route") != ("fused_xa" if fused_xa else "plain"):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(spec, d0, Ts, optimizer="sgd", frozen=False, g_fmt="e4m3", x_note="",
                 min_seconds=10.0, one_thread_tokens=512, one_thread_seconds=5.0):
    """The CPU oracle, as it is, on a token sample of the same workload:
    quantize X and dY, forward, backward (dX, dA, dB; or with A frozen in FP8,
    X~A~^T in the forward and dX, dB), the adapter step (SGD or AdamW) and
    the proxy update over the full backbone; the step is repeated on the same
    inputs until `min_seconds` have passed, and the mean is reported.  Then
    the same on one host thread (BLAS and the C part limited to one), on
    the first `one_thread_tokens` tokens (0: skipped)."""
    import numpy as np

    import oracle
    import workloads as wl

    t0 = time.perf_counter()
    wq, s_w, _, _ = oracle.fp8_quantize(d0["W"])
    A0 = d0["A"]
    aq = s_a = None
    if frozen:
        aq, s_a, _, _ = oracle.fp8_quantize(A0)
        A0 = oracle.fp8_dequantize(aq, s_a)
    t_init = time.perf_counter() - t0

    def timed(n_tok, seconds):
        X = d0["X"][:n_tok]
        dY = d0["dY"][:n_tok]
        t1 = time.perf_counter()
        reps = 0
        while True:
            _oracle_step(oracle, np, spec, X, dY, wq, s_w, A0, d0["B"], aq, s_a, optimizer,
                         frozen, g_fmt)
            reps += 1
            if time.perf_counter() - t1 >= seconds:
                break
        return (time.perf_counter() - t1) / reps, reps

    step_s, reps = timed(Ts, min_seconds)
    flops = wl.step_flops(Ts, spec.d_in, spec.d_out, spec.rank, frozen_a=frozen)
    try:
        import threadpoolctl
        blas = threadpoolctl.threadpool_info()
        blas_threads = max([b.get("num_threads", 1) for b in blas] or [1])
    except Exception:
        threadpoolctl = None
        blas_threads = os.cpu_count()
    out = {"value": round(flops / step_s / 1e12, 5), "unit": "TFLOP/s", "cores": int(max(
        blas_threads, oracle.num_threads())), "kind": "oracle",
        "tokens_per_s": round(Ts / step_s, 1),
        "sample": f"the step on the first {Ts} of {spec.tokens} tokens{x_note} (full "
                  f"{spec.d_out} x {spec.d_in} weight, r={spec.rank}, full proxy update), "
                  f"{reps} repetition{'s' if reps > 1 else ''}, mean {step_s:.2f} s; the "
                  f"initial quantization of W{' and A' if frozen else ''} ({t_init:.1f} s) "
                  f"is not part of the step"}
    n1 = min(one_thread_tokens, Ts)
    if n1 > 0 and threadpoolctl is not None:
        threads = oracle.num_threads()
        with threadpoolctl.threadpool_limits(limits=1):
            oracle.set_num_threads(1)
            try:
                s1, reps1 = timed(n1, one_thread_seconds)
            finally:
                oracle.set_num_threads(threads)
        f1 = wl.step_flops(n1, spec.d_in, spec.d_out, spec.rank, frozen_a=frozen)
        out["one_thread"] = {
            "value": round(f1 / s1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "tokens_per_s": round(n1 / s1, 1),
            "sample": f"the same step on the first {n1} tokens, BLAS and OpenMP limited to one "
                      f"thread, {reps1} repetition{'s' if reps1 > 1 else ''}, mean {s1:.2f} s"}
    return out


def _oracle_step(oracle, np, spec, X, dY, wq, s_w, A0, B0, aq, s_a, optimizer, frozen, g_fmt):
    """one step of the oracle from the given state (nothing is kept)"""
    xq, s_x, _, _ = oracle.fp8_quantize(X)
    gq, s_g, _, _ = oracle.fp8_quantize(dY, fmt=g_fmt)
    if frozen:
        _, U = oracle.melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a)
        _, dB = oracle.melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, U, g_fmt=g_fmt)
        dA = None
    else:
        oracle.melded_linear_fwd(xq, s_x, wq, s_w)
        _, dA, dB = oracle.melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A0, B0, g_fmt=g_fmt)
    if optimizer == "sgd":
        A, B = oracle.adapter_step(A0, B0, dA, dB, spec.lr)
    else:
        z = [np.zeros_like(A0), np.zeros_like(B0)]
        A, B, _, _, _, _ = oracle.adapter_step_adamw(A0, B0, dA, dB, z[0], z[0], z[1],
                                                     z[1], spec.lr, 0.9, 0.999, 1e-8, 0.0, 1)
    oracle.rowwise_proxy_update(wq, s_w, A, B, spec.tau, spec.k_max)


if __name__ == "__main__":
    main()
