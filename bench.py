#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

Workload: the concurrency-sweep MoE layer -- hidden 7168, 256 routed experts, top-8, expert SwiGLU
intermediate 2048, MXFP4 expert weights (codes uniform, E8M0 in [118, 127]), bf16 activations
~N(0,1), router weights ~N(0, 1/7168) so logits are ~N(0,1); seeded synthetic inputs (seed 0).
One step = one layer call on T tokens (default 176): moe_route_bucket (router, bucketing and the
expert FFN's tile plan) -> moe_expert_ffn_gateup -> moe_expert_ffn_down -> moe_combine, inputs resident
in HBM.  Weight sets are rotated so that the bytes touched between two visits of one set exceed the
256 MB Infinity Cache (a one-set control is reported where rotation applies).  The rotated copies
are made once and, like every other buffer, freed only after the last GPU measurement: device memory
freed during the run is cleared by the driver in the background, and that traffic slowed the
kernels timed in the next seconds by about 3%.

Each T is timed twice: eager (the library calls issued from Python, HIP events around the steps and
between the calls) and replayed from HIP graphs that hold one layer call each (the headline: the
host's launch work is then out of the loop, which matters at small T); the graph pass also gives
the per-step p10 / median / p90.

Prints one JSON line: tokens/s (value, graph replay), ms per layer call, the gate/up kernel's
roofline (HIP-event duration and algorithmic bytes), the per-T sweep T = 1..176, a measured
read-stream peak beside the nominal 8 TB/s, the prefill layer (T = 8192, exact and MX-FP6 modes,
fraction of the MXFP4 MFMA peak), and the fp64 CPU oracle timed on bounded samples.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
INFINITY_CACHE = 256 << 20
MXFP4_BYTES_PER_WEIGHT = 17.0 / 32.0   # 4.25 bits


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--tokens", type=int, default=176, help="T of the headline step")
    ap.add_argument("--sweep-steps", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16, help="tokens of the oracle's timed sample")
    ap.add_argument("--prefill", action="store_true",
                    help="measure the prefill layer instead (T=8192, 256 routed + 1 shared expert, top-8, "
                         "log-Zipf routing bias) and print its own JSON line with MFMA utilisation")
    ap.add_argument("--mx", choices=["fp8", "fp6", "fp4"], default=None,
                    help="with --prefill: the MX mode of the expert FFN (activations quantised to MXFP8 E4M3, "
                         "MXFP6 E2M3 or MXFP4 E2M1 and multiplied with the FP4 weights on scaled MFMAs)")
    ap.add_argument("--workload", choices=["decode", "dense"], default=None,
                    help="measure another layer workload instead and print its own JSON line: the decode "
                         "layer (hidden 4096, 128 experts, top-8, I 1536, MXFP4; T = 1, 8, 32, 64) or the "
                         "dense FFN as 8 all-active FP16 slices (hidden 4096, I 16384; T = 1, 16, 128)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave the prefill object (T=8192, exact and MX-FP6 expert FFN) out of the default line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain elementwise copy (torch.neg, fp32) of this many MiB three times, "
                         "for scaling memory counters, and exit")
    return ap.parse_args()


class Runner:
    """Preallocated buffers for one T; step(set) enqueues the five library calls on the current stream."""

    def __init__(self, moe, sets, T, top_k, n_shared, n_experts, H, I, mx=None, fixed_routing=False):
        import torch
        dev = "cuda:0"
        self.moe, self.sets, self.T, self.top_k, self.n_shared = moe, sets, T, top_k, n_shared
        self.mx = mx
        self.fixed = fixed_routing  # dense slices: ids [t][j] = j, weights 1, no router call
        self.fused = mx is None and not fixed_routing
        self.kt = top_k + n_shared
        self.n_experts = n_experts
        n = T * self.kt
        W0 = sets[0]["W"]
        self.ids = torch.empty((T, self.kt), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, self.kt), dtype=torch.float32, device=dev)
        if fixed_routing:
            self.ids.copy_(torch.arange(self.kt, dtype=torch.int32, device=dev).expand(T, self.kt))
            self.w.fill_(1.0)
        self.route_ws = None if fixed_routing else self._ws(
            moe.moe_route_bucket_workspace_bytes(T, H, n_experts - n_shared, top_k, n_shared))
        self.b = moe.Buckets(torch.empty(n_experts, dtype=torch.int32, device=dev),
                             torch.empty(n_experts + 1, dtype=torch.int32, device=dev),
                             torch.empty(n, dtype=torch.int32, device=dev), None)
        self.bucket_ws = self._ws(moe.moe_bucket_workspace_bytes(n, n_experts))
        self.ffn_ws = self._ws(moe.moe_expert_ffn_workspace_bytes(T, self.kt, W0) if mx is None
                               else moe.moe_expert_ffn_mx_workspace_bytes(T, self.kt, W0, mx))
        self.y_slots = torch.empty((n, H), dtype=torch.float32, device=dev)
        self.y = torch.empty((T, H), dtype=torch.float32, device=dev)

    @staticmethod
    def _ws(nbytes):
        import torch
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda:0")

    def step(self, i, events=None):
        m, s = self.moe, self.sets[i % len(self.sets)]
        rec = (lambda k: events[k].record()) if events is not None else (lambda k: None)
        if self.fused:
            # router + bucketing + tile plan in one call (two launches), then gate/up, down, combine
            rec(0)
            m.moe_route_bucket(s["x"][:self.T], s["router"], self.top_k, s["bias"], self.n_shared, self.ids, self.w,
                               self.b, s["W"], self.ffn_ws, workspace=self.route_ws)
            rec(1)
            rec(2)
            rec(3)
            m.moe_expert_ffn_gateup(s["x"][:self.T], s["W"], self.b.offsets, self.b.sorted_slot, self.kt, self.ffn_ws)
            rec(4)
            m.moe_expert_ffn_down(self.T, s["W"], self.b.offsets, self.b.sorted_slot, self.kt, self.ffn_ws,
                                  self.y_slots)
            rec(5)
            m.moe_combine(self.y_slots, self.w, out=self.y)
            rec(6)
            return
        rec(0)
        if not self.fixed:
            m.moe_route(s["x"][:self.T], s["router"], self.top_k, s["bias"], self.n_shared,
                        out=(self.ids, self.w, None), workspace=self.route_ws)
        rec(1)
        m.moe_bucket(self.ids, self.n_experts, out=self.b, workspace=self.bucket_ws)
        rec(2)
        if self.mx is not None:  # MX mode: one call (x quantisation, plan, gate/up, down)
            m.moe_expert_ffn_mx(s["x"][:self.T], s["W"], self.mx, self.b.offsets, self.b.sorted_slot, self.kt,
                                out=self.y_slots, workspace=self.ffn_ws)
            rec(3)
            rec(4)
        else:
            m.moe_expert_ffn_plan(self.T, s["W"], self.b.offsets, self.kt, self.ffn_ws)
            rec(3)
            m.moe_expert_ffn_gateup(s["x"][:self.T], s["W"], self.b.offsets, self.b.sorted_slot, self.kt,
                                    self.ffn_ws)
            rec(4)
            m.moe_expert_ffn_down(self.T, s["W"], self.b.offsets, self.b.sorted_slot, self.kt, self.ffn_ws,
                                  self.y_slots)
        rec(5)
        m.moe_combine(self.y_slots, self.w, out=self.y)
        rec(6)


def time_steps(runner, steps, warmup):
    """-> (ms per step from events around all steps, per-call mean ms from per-step events)."""
    import torch
    for i in range(warmup):
        runner.step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        runner.step(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end) / steps
    # second timed pass with events between the calls (same stream, same kernels)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    for i in range(steps):
        runner.step(i, evs[i])
    torch.cuda.synchronize()
    names = (["route_bucket_plan", None, None, "ffn_gateup", "ffn_down", "combine"] if runner.fused else
             ["route", "bucket", "ffn_plan", "ffn_gateup", "ffn_down", "combine"])
    per = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(names) if n}
    return total_ms, per


def time_graph(runner, steps, warmup):
    """The same steps replayed from HIP graphs, one graph per rotated weight set (one layer call
    each), so host-side launch work is out of the loop -> ms per step."""
    import torch
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(len(runner.sets)):
            runner.step(i)                      # eager pass on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(len(runner.sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            runner.step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    mean_ms = start.elapsed_time(end) / steps
    # a second pass with an event between consecutive replays: the per-step distribution
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    q = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    del graphs
    return mean_ms, {"p10": q(0.1), "median": q(0.5), "p90": q(0.9)}


def active_experts(runner):
    import torch
    torch.cuda.synchronize()
    return int((runner.b.counts.cpu() > 0).sum().item())


def traffic_record(kernel_src):
    """FETCH/WRITE bytes per launch of the gate/up kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "ffn_gateup_T176_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    digest = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != digest:
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this layer build has no "
              "multi-GPU path: see the sharding design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration_mib:
        return copy_calibration(args.copy_calibration_mib)
    if args.prefill:
        return prefill_run(args)
    if args.workload:
        return side_run(args)
    import synth
    import mxfp4_routed_expert_router_amd as moe

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    wl = synth.WORKLOADS["sweep"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_routed, wl.top_k
    Ts = sorted(set(([] if args.no_sweep else list(wl.tokens)) + [args.tokens]))
    Tmax = max(Ts)
    t0 = time.time()
    L = synth.make_layer(wl, Tmax)
    base = synth.to_torch(L, "cuda:0")
    gen_s = time.time() - t0
    expert_bytes = 3 * H * I * MXFP4_BYTES_PER_WEIGHT

    def n_sets(T):
        # enough independent copies (router + weights) that one pass over them exceeds 4x the cache
        a = E * (1.0 - (1.0 - k / E) ** T)
        return max(1, min(16, math.ceil(4 * INFINITY_CACHE / (a * expert_bytes + 4 * H * E))))

    pool = weight_pool(moe, base, max(n_sets(T) for T in Ts))
    results = {}
    for T in Ts:
        print(f"bench: T={T}", file=sys.stderr, flush=True)
        sets = pool[:n_sets(T)]
        runner = Runner(moe, sets, T, k, 0, E, H, I)
        steps = args.steps if T == args.tokens else args.sweep_steps
        warm = args.warmup if T == args.tokens else min(args.warmup, 5)
        eager_ms, per = time_steps(runner, steps, warm)
        graph_ms, dist = time_graph(runner, steps, warm)
        ms = graph_ms
        A = active_experts(runner)
        n_slots = T * k
        w_bytes = A * expert_bytes
        gateup_bytes = A * 2 * H * I * MXFP4_BYTES_PER_WEIGHT + n_slots * (2 * H + 4 * I)
        results[T] = dict(T=T, ms=ms, eager_ms=eager_ms, per=per, dist=dist, active=A, weight_bytes=w_bytes,
                          gateup_bytes=gateup_bytes, rotation_sets=len(sets), steps=steps)
        if len(sets) > 1:
            # control: the same calls on one weight set, which then stays in the Infinity Cache
            runner.sets = sets[:1]
            results[T]["no_rotation_ms"] = time_graph(runner, steps, warm)[0]
        del runner, sets

    print("bench: read-stream peak", file=sys.stderr, flush=True)
    read_peak, plain_read, read_buf = read_stream_peak()

    head = results[args.tokens]
    t_gu = head["per"]["ffn_gateup"] / 1e3
    achieved = head["gateup_bytes"] / t_gu
    traffic = traffic_record(os.path.join(ROOT, "mxfp4_routed_expert_router_amd", "csrc", "ffn.hip"))
    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (MXFP4 expert weights), T=1..176",
        "value": args.tokens / (head["ms"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"moe_layer_sweep_H7168_E256_top8_I2048_mxfp4_T{args.tokens}",
                   "tokens": args.tokens, "hidden": H, "routed_experts": E, "top_k": k, "inter": I,
                   "weights": "mxfp4 (E2M1 + E8M0/32)", "activations": "bf16", "output": "fp32",
                   "parallelism": "single GPU", "timing": "HIP graph replay of whole layer calls"},
        "eager_ms_per_step": head["eager_ms"],
        "ms_per_step_p10_median_p90": [head["dist"]["p10"], head["dist"]["median"], head["dist"]["p90"]],
        "weight_GBps": head["weight_bytes"] / (head["ms"] / 1e3) / 1e9,
        "weight_frac_of_hbm_peak": head["weight_bytes"] / (head["ms"] / 1e3) / HBM_PEAK,
        "read_stream_peak_GBps": read_peak / 1e9,
        "plain_read_GBps": plain_read / 1e9,
        "weight_frac_of_read_stream_peak": head["weight_bytes"] / (head["ms"] / 1e3) / read_peak,
        "active_experts": head["active"],
        "rotation_sets": head["rotation_sets"],
        "per_call_ms": {kk: round(v, 5) for kk, v in head["per"].items()},
        "roofline": {"kernel": "ffn_gateup_rows_kernel (moe_expert_ffn_gateup: grouped MXFP4 gate/up GEMM + SwiGLU)",
                     "bound": "hbm",
                     "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": traffic,
                     "traffic_source": ("stored rocprofv3 --pmc record (FETCH_SIZE + WRITE_SIZE per launch, "
                                        "profiles/ffn_gateup_T176_counters.json), valid for the current ffn.hip "
                                        "source" if traffic is not None else
                                        "none: the stored counter record predates the current ffn.hip source"),
                     "frac_of_read_stream_peak": achieved / read_peak,
                     "algorithmic_bytes_per_launch": head["gateup_bytes"], "launch_ms": head["per"]["ffn_gateup"]},
        "sweep": [{"T": r["T"], "us_per_layer": r["ms"] * 1e3, "eager_us_per_layer": r["eager_ms"] * 1e3,
                   "us_p10_median_p90": [r["dist"]["p10"] * 1e3, r["dist"]["median"] * 1e3, r["dist"]["p90"] * 1e3],
                   "tokens_per_s": r["T"] / (r["ms"] / 1e3),
                   "active_experts": r["active"], "weight_GBps": r["weight_bytes"] / (r["ms"] / 1e3) / 1e9,
                   "weight_frac_of_hbm_peak": r["weight_bytes"] / (r["ms"] / 1e3) / HBM_PEAK,
                   "gateup_us": r["per"]["ffn_gateup"] * 1e3, "down_us": r["per"]["ffn_down"] * 1e3,
                   "rotation_sets": r["rotation_sets"],
                   **({"no_rotation_us_per_layer": r["no_rotation_ms"] * 1e3} if "no_rotation_ms" in r else {})}
                  for r in (results[T] for T in Ts)],
        "input_generation_s": gen_s,
    }
    pre_L = None
    if not args.no_prefill:
        print("bench: prefill", file=sys.stderr, flush=True)
        out["prefill"], pre_L = prefill_measure(max(2, args.warmup // 3), 5)
    # nothing is freed before the last GPU measurement: the driver clears freed device memory in
    # the background, and that traffic slows the kernels measured next (about 3% for several
    # seconds after freeing the rotated weight sets)
    del pool, base, read_buf
    if not args.no_cpu:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(L, args.tokens, args.cpu_tokens, pre_L)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def weight_pool(moe, base, n, fix=None):
    """n weight sets: the inputs `base` and n - 1 copies of them, allocated once and kept until the
    measurements end (fix(t) adjusts a copy's views, e.g. the dense slices)."""
    sets = []
    for j in range(n):
        if j == 0:
            t = base
        else:
            t = {kk: (v.clone() if hasattr(v, "clone") else v) for kk, v in base.items()}
            if fix is not None:
                fix(t)
        W = moe.ExpertWeights(t["gate"], t["gate_scales"], t["up"], t["up_scales"], t["down"], t["down_scales"])
        sets.append({"x": t["x"], "router": t["router"], "bias": t["bias"], "W": W, "t": t})
    return sets


def read_stream_peak(gib=4, reps=5):
    """Practical read bandwidth of this chip in this process, beside the nominal 8 TB/s, in two forms
    over one 4 GiB buffer (best of reps each):
      line -- moe_stream_read: the library's streaming read with 16-byte nontemporal loads covering
              whole 128-byte lines per wave load, the shape the streaming FFN kernels read their
              weights in; this is the peak the kernels are compared with;
      plain -- torch row sums of 4096 consecutive fp32 values (every row one contiguous 16 KB
              read), an ordinary cached read.
    (A single whole-buffer torch.sum reads slower, about 4 TB/s: its reduction tree, not memory,
    limits it.)  Returns (line, plain, buffer); the caller frees the buffer once nothing else is
    timed."""
    import torch
    import mxfp4_routed_expert_router_amd as moe
    n = (gib << 30) // 4
    buf = torch.ones(n, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    rows = buf.view(-1, 4096)

    def best_of(fn):
        fn()
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            best = max(best, n * 4 / (a.elapsed_time(b) / 1e3))
        return best

    line = best_of(lambda: moe.moe_stream_read(buf, sink))
    plain = best_of(lambda: rows.sum(1))
    return line, plain, buf


def side_run(args):
    """The decode or dense-slices workload at each of its token counts (its own JSON line; weight
    sets rotated past the Infinity Cache as in the sweep)."""
    import torch
    import synth
    import mxfp4_routed_expert_router_amd as moe
    moe.lib()
    name = "decode" if args.workload == "decode" else "dense_slices"
    wl = synth.WORKLOADS[name]
    H, I, E, k = wl.hidden, wl.inter, wl.n_routed, wl.top_k
    dense = wl.dense_slices
    Ts = list(wl.tokens)
    t0 = time.time()
    L = synth.make_layer(wl, max(Ts))
    base = synth.to_torch(L, "cuda:0")
    gen_s = time.time() - t0
    expert_bytes = 3 * H * I * (2.0 if dense else MXFP4_BYTES_PER_WEIGHT)

    def n_sets(T):
        a = E if dense else E * (1.0 - (1.0 - k / E) ** T)
        return max(1, min(16, math.ceil(4 * INFINITY_CACHE / (a * expert_bytes))))

    def slices(t):  # keep the slice views over the copied dense matrices
        E2 = wl.n_experts
        t["gate"], t["up"] = t["dense_gate"].view(E2, I, H), t["dense_up"].view(E2, I, H)
        t["down"] = t["dense_down"].as_strided((E2, H, I), (I, E2 * I, 1))

    pool = weight_pool(moe, base, max(n_sets(T) for T in Ts), slices if dense else None)
    lines = []
    for T in Ts:
        print(f"bench {name}: T={T}", file=sys.stderr, flush=True)
        sets = pool[:n_sets(T)]
        runner = Runner(moe, sets, T, k, 0, E, H, I, fixed_routing=dense)
        eager_ms, per = time_steps(runner, args.sweep_steps, min(args.warmup, 5))
        ms, dist = time_graph(runner, args.sweep_steps, min(args.warmup, 5))
        A = E if dense else active_experts(runner)
        wb = A * expert_bytes
        lines.append({"T": T, "us_per_layer": ms * 1e3, "eager_us_per_layer": eager_ms * 1e3,
                      "us_p10_median_p90": [dist["p10"] * 1e3, dist["median"] * 1e3, dist["p90"] * 1e3],
                      "tokens_per_s": T / (ms / 1e3), "active_experts": A, "weight_GBps": wb / (ms / 1e3) / 1e9,
                      "weight_frac_of_hbm_peak": wb / (ms / 1e3) / HBM_PEAK,
                      "per_call_us": {kk: round(v * 1e3, 2) for kk, v in per.items()},
                      "rotation_sets": len(sets)})
        del runner, sets
    wdesc = "fp16 (8 all-active slices of one dense FFN)" if dense else "mxfp4 (E2M1 + E8M0/32)"
    out = {"metric": f"{name} MoE-layer tokens/s and HBM GB/s on expert weights (side measurement)",
           "n_gpus": 1, "data": "synthetic", "higher_is_better": True,
           "config": {"workload": f"moe_layer_{name}_H{H}_E{E}_top{k}_I{I}", "hidden": H, "experts": E,
                      "top_k": k, "inter": I, "weights": wdesc, "activations": wl.act_dtype, "output": "fp32",
                      "timing": "HIP graph replay of whole layer calls"},
           "sweep": lines, "input_generation_s": gen_s}
    print(json.dumps(out), flush=True)


def prefill_inputs():
    """The prefill layer's inputs on the GPU (one weight set: its 6 GB of expert weights exceed the
    Infinity Cache many times over)."""
    import synth
    import mxfp4_routed_expert_router_amd as moe
    moe.lib()
    wl = synth.WORKLOADS["prefill"]
    t0 = time.time()
    L = synth.make_layer(wl, wl.tokens[0])
    t = synth.to_torch(L, "cuda:0")
    W = moe.ExpertWeights(t["gate"], t["gate_scales"], t["up"], t["up_scales"], t["down"], t["down_scales"])
    return wl, [{"x": t["x"], "router": t["router"], "bias": t["bias"], "W": W, "t": t}], time.time() - t0, L


def prefill_mode(wl, sets, mx, steps, warmup):
    """One prefill mode (exact: mx None; else the MX activation format) -> timing record."""
    import mxfp4_routed_expert_router_amd as moe
    T = wl.tokens[0]
    H, I, E, k, S = wl.hidden, wl.inter, wl.n_routed, wl.top_k, wl.n_shared
    runner = Runner(moe, sets, T, k, S, E + S, H, I, mx=mx)
    ms, per = time_steps(runner, steps, warmup)
    counts = runner.b.counts.cpu()
    kt = k + S
    ffn_flops = 6.0 * H * I * T * kt
    ffn_ms = sum(per.get(kk, 0.0) for kk in ("ffn_plan", "ffn_gateup", "ffn_down")) if mx is not None else \
        per["ffn_gateup"] + per["ffn_down"]
    rec = {"mode": "exact" if mx is None else f"mx_{mx}", "ms_per_layer": ms, "tokens_per_s": T / (ms / 1e3),
           "ffn_ms": ffn_ms, "ffn_tflops": ffn_flops / (ffn_ms / 1e3) / 1e12,
           "frac_of_bf16_mfma_peak": ffn_flops / (ffn_ms / 1e3) / 2.5e15,
           "frac_of_mxfp4_mfma_peak": ffn_flops / (ffn_ms / 1e3) / 10.1e15,
           "active_experts": int((counts > 0).sum().item()), "max_rows_per_expert": int(counts.max().item()),
           "per_call_ms": {kk: round(v, 4) for kk, v in per.items()}}
    if mx is None:
        rec["gateup_tflops"] = 4.0 * H * I * T * kt / (per["ffn_gateup"] / 1e3) / 1e12
        rec["down_tflops"] = 2.0 * H * I * T * kt / (per["ffn_down"] / 1e3) / 1e12
    else:
        rec["per_call_ms"]["ffn_mx"] = rec["per_call_ms"].pop("ffn_plan")
        for kk in ("ffn_gateup", "ffn_down"):  # one call: its kernels are split by the profiler only
            rec["per_call_ms"].pop(kk)
    del runner
    return rec


def prefill_measure(warmup, steps):
    """The prefill object of the default line: T = 8192, exact mode and MX mode with MXFP6
    activations, FFN time and the fraction of the MXFP4 MFMA peak (10.1 PFLOP/s)."""
    import torch
    wl, sets, gen_s, L = prefill_inputs()
    out = {"workload": f"moe_layer_prefill_H{wl.hidden}_E{wl.n_routed}+{wl.n_shared}_top{wl.top_k}_I{wl.inter}"
                       f"_mxfp4_T{wl.tokens[0]}", "input_generation_s": gen_s}
    for mx in (None, "fp6"):
        out["exact" if mx is None else f"mx_{mx}"] = prefill_mode(wl, sets, mx, steps, warmup)
    del sets
    return out, L


def prefill_run(args):
    """The prefill layer alone (its own JSON line).  Exact mode: weights decoded to bf16 in
    registers, bf16 MFMA with fp32 accumulation, h as a bf16 hi + lo pair (two MFMAs per down
    product); MX mode with --mx."""
    wl, sets, gen_s, _ = prefill_inputs()
    T = wl.tokens[0]
    H, I, E, k, S = wl.hidden, wl.inter, wl.n_routed, wl.top_k, wl.n_shared
    rec = prefill_mode(wl, sets, args.mx, args.steps, args.warmup)
    mode = "exact mode" if args.mx is None else f"MX mode, {args.mx} activations"
    out = {
        "metric": f"prefill MoE-layer tokens/s and MFMA utilisation ({mode})",
        "value": rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": rec["ms_per_layer"], "higher_is_better": True,
        "dtype": "bf16" if args.mx is None else f"fp4 weights x {args.mx} activations", "data": "synthetic",
        "config": {"workload": f"moe_layer_prefill_H{H}_E{E}+{S}_top{k}_I{I}_mxfp4_T{T}", "tokens": T,
                   "zipf_s": wl.zipf_s, "mode": rec["mode"]},
        "layer_flops": 6.0 * H * I * T * (k + S) + 2.0 * T * H * E,
        "input_generation_s": gen_s,
    }
    out.update({kk: v for kk, v in rec.items() if kk not in ("mode", "ms_per_layer", "tokens_per_s")})
    print(json.dumps(out), flush=True)


def copy_calibration(mib):
    """A plain device copy of known size (reads and writes mib MiB each), to scale FETCH_SIZE and
    WRITE_SIZE readings into bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(L, T, n, pre=None):
    """The fp64 oracle as it stands, timed on the host cores (OpenMP over its default thread count,
    plus one single-thread run).  `value`: the first n tokens of the benchmark's own T-token batch
    run as one n-token layer call (route, bucket, grouped expert FFN, combine).  `runs`: the other
    layer workloads -- the tiny layer (median of 5, all threads and one thread), the decode layer at
    T = 8, the dense FFN as 8 all-active FP16 slices at T = 1, and the prefill layer, whose routing
    and bucketing run on all 8192 tokens while its expert FFN runs on 8 tokens and is extrapolated
    per token to the batch (labelled as such)."""
    import dataclasses
    import statistics
    import numpy as np
    import oracle
    import synth
    o = oracle.load()
    threads = o.num_threads()
    sub = dataclasses.replace(L, T=n, x=L.x[:n])
    t0 = time.perf_counter()
    o.layer(sub)
    dt = time.perf_counter() - t0
    runs = []

    def timed(fn, reps=1):
        ts = []
        for _ in range(reps):
            a = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - a)
        return statistics.median(ts)

    tiny = synth.make_layer(synth.WORKLOADS["tiny"], 16)
    t_all = timed(lambda: o.layer(tiny), 5)
    o.set_num_threads(1)
    t_one = timed(lambda: o.layer(tiny), 5)
    o.set_num_threads(threads)
    runs.append({"workload": "tiny T=16", "s_per_layer": t_all, "tokens_per_s": 16 / t_all, "threads": threads,
                 "stat": "median of 5"})
    runs.append({"workload": "tiny T=16", "s_per_layer": t_one, "tokens_per_s": 16 / t_one, "threads": 1,
                 "stat": "median of 5"})
    dec = synth.make_layer(synth.WORKLOADS["decode"], 8)
    t_dec = timed(lambda: o.layer(dec))
    runs.append({"workload": "decode T=8", "s_per_layer": t_dec, "tokens_per_s": 8 / t_dec, "threads": threads})
    dense = synth.make_layer(synth.WORKLOADS["dense_slices"], 1)
    t_den = timed(lambda: o.layer(dense))
    runs.append({"workload": "dense_slices T=1", "s_per_layer": t_den, "tokens_per_s": 1 / t_den,
                 "threads": threads})
    wl = synth.WORKLOADS["prefill"]
    if pre is None:
        pre = synth.make_layer(wl, wl.tokens[0])
    a = time.perf_counter()
    r = o.route(pre.x, oracle.X_BF16, pre.router, pre.bias, wl.top_k, wl.n_shared)
    o.bucket(r["ids"], wl.n_experts)
    t_rb = time.perf_counter() - a
    mask = np.zeros(pre.T, np.uint8)
    mask[np.linspace(0, pre.T - 1, 8).astype(int)] = 1
    t_ffn8 = timed(lambda: o.layer(pre, token_mask=mask))
    runs.append({"workload": "prefill T=8192 route + bucket (all tokens)", "s": t_rb, "threads": threads})
    runs.append({"workload": "prefill T=8192 whole layer", "extrapolated": True,
                 "s_per_layer": t_rb + (t_ffn8 - t_rb) * pre.T / 8, "threads": threads,
                 "how": "route + bucket measured on all 8192 tokens; expert FFN and combine measured on 8 spread "
                        "tokens (that call also re-routes all tokens) and scaled by 8192 / 8"})
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of the {T}-token batch as one {n}-token layer call (route, bucket, expert FFN, "
                      f"combine in fp64); {dt:.1f} s",
            "cpu_model": cpu_model(), "hardware_threads": os.cpu_count(), "runs": runs}


if __name__ == "__main__":
    main()
