#!/usr/bin/env python3
"""Benchmark of the fused MoE expert FFN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload skewed]

The default workload is skewed (16,384 tokens, hidden 7168, intermediate 2048, 32 local experts of
256, Zipf(1.2) top-8 routing, 10% of the rows of x scaled by 50): the largest of the configurations
that fits one GPU, the one the headline number is quoted on.

One step = the whole hot path on one batch of synthetic input already resident
in HBM: routing tables (moe_plan), grouped Linear1 with the fused
SwiGLU/requant epilogue, grouped Linear2, and the top-k combine, enqueued on
one stream.  The stages are the calls moe_forward makes (moe_plan,
moe_expert_ffn, both GEMMs in one persistent launch, or moe_linear1 and
moe_linear2, as moe_gemm_launches reports; moe_combine); they are issued one by one so HIP
events on that stream can bracket the dominant GEMM launch inside the timed
steps (the roofline's achieved rate; on every fourth timed step by default,
--event-every).  Each call's arguments are checked and marshalled once
before the timed loop (binding.Bound).  --forward times whole moe_forward
calls instead (the plan built inside the workspace), the events then
bracketing the whole forward.  --staged and --expert-ffn force one
schedule or the other.  In the two-launch schedule every timed step is
recorded as three HIP graphs (the calls before the dominant GEMM launch, that
launch, the calls after it) and the timed loop replays them, recording the
events around the dominant launch between the replays; the single-launch
schedule issues the calls one by one on the stream (--launch graph or stream
forces either).  Three copies of the
expert weights are rotated between steps so they stream from HBM rather than
the 256 MB Infinity Cache.  The default warmup (50 steps) lets the clocks
settle; the first steps after idle run ~15% slower.

Prints one JSON line with the metric (useful TFLOP/s = 2 * N_valid * 3 * H * I
per step, the reading notes' FLOP count, over the wall time of the timed
steps), tokens/s, the share of the step's compulsory HBM bytes per second in
the HBM peak, the roofline of the dominant kernel (MFMA or HBM, whichever
bounds its algorithmic work), per-stage kernel times
from a separate untimed pass with an event between every stage, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer useful TFLOP/s + tokens/s at 1 GPU; % of scaled-MFMA peak / HBM BW"
PEAK_MFMA_TFLOPS = 5000.0      # MI355X dense FP8 MFMA; FP8 x FP4 scaled MFMA issues at this rate
PEAK_HBM_GBS = 8000.0


class DeviceEvents:
    """HIP events created with hipEventDisableSystemFence, for timing only.  A default event performs a
    system-scope memory fence when it completes (a writeback and invalidation of the caches), which on
    this GPU costs the kernels that follow it time; these events record the timestamp without it.  They
    come from the HIP runtime torch has loaded, so torch's stream handles are valid for them."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def new(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(e)
        return e

    def record(self, e, stream):
        """Record on `stream` (not inside a graph capture: the timed graph replays record their events
        between the replays)."""
        import torch
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("bench.py: timing events are recorded between graph replays, not captured")
        rc = self.hip.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        """Milliseconds between two recorded events; the stream must have been synchronized."""
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def kernel_traffic(kind: str, workload: str):
    """HBM bytes per launch of the dominant GEMM kernel (kind: expert_ffn or linear1) from the committed
    rocprofv3 byte-counter summary, when it was taken on this workload with the current GEMM source (its
    sha256 is recorded there); else None."""
    path = os.path.join(ROOT, "profiles", f"{kind}_gemm_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip()
    src = os.path.join(ROOT, "moe_expert_ffn_plan_amd", "csrc", "moe_gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest or fields.get("workload") != workload:
        return None
    return int(fields["traffic_bytes_per_launch"])


def kernel_bytes(w, fused: bool, n_valid: int, touched: int, hit_tokens: int) -> int:
    """Algorithmic HBM bytes of one launch of the dominant GEMM kernel: what it must read and write once.
    Linear1: W1 and its scales for every expert with a row, x and x_sf of every token with a local hit,
    one top-k weight per row, h_q and h_sf written.  Both GEMMs in one launch: that, plus W2 and its
    scales for the same experts, h_q and h_sf read back, and the BF16 yslot rows written."""
    H, I = w.hidden, w.intermediate
    w1 = touched * 2 * I * H * (1 / 2 + 1 / 32)
    h = n_valid * I * (1 + 1 / 32)
    b = w1 + hit_tokens * H * (1 + 1 / 32) + n_valid * 4 + h
    if fused:
        b += touched * H * I * (1 / 2 + 1 / 32) + h + n_valid * H * 2
    return int(b)


def cpu_baseline(w, d_gpu, sample_tokens: int, min_seconds: float = 10.0):
    """Time the CPU oracle (untuned) on the first `sample_tokens` tokens of the workload, repeated until
    at least `min_seconds` have passed."""
    import numpy as np
    from moe_expert_ffn_plan_amd import inputs
    from oracle.forward import forward_tokens
    d = inputs.to_numpy(d_gpu)
    toks = np.arange(min(sample_tokens, w.num_tokens))
    reps, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        _, hits = forward_tokens(toks, d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"],
                                 d["w2"], d["w2_sf"], num_experts=w.num_experts, expert_begin=0)
        dt += time.perf_counter() - t0
        reps += 1
    flops = 2.0 * len(hits) * 3 * w.hidden * w.intermediate * reps
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max(int(i.get("num_threads", 1)) for i in pools) or 1
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')}, "
                         f"{i.get('num_threads')} threads)" for i in pools)
    except Exception:
        cores = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"first {toks.size} of {w.num_tokens} tokens ({len(hits)} local top-k rows), whole oracle "
                      f"forward incl. weight dequantisation, {reps} run(s), {dt:.1f} s",
            "cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas": blas}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="skewed")
    ap.add_argument("--weight-copies", type=int, default=3)
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--staged", action="store_true",
                    help="run Linear1 and Linear2 as two launches (moe_linear1, moe_linear2) for every shape")
    ap.add_argument("--expert-ffn", action="store_true",
                    help="run Linear1 and Linear2 through moe_expert_ffn (one launch) wherever it is supported")
    ap.add_argument("--forward", action="store_true",
                    help="time whole moe_forward calls (the plan built inside the workspace, one call per step); "
                         "the events then bracket the whole forward and the roofline is the step's")
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the events around the dominant launch on every N-th timed step (default 4)")
    ap.add_argument("--host-inputs", action="store_true",
                    help="draw the synthetic inputs on the CPU and copy them (fewer torch GPU kernels, for profilers)")
    ap.add_argument("--launch", choices=("auto", "graph", "stream"), default="auto",
                    help="graph: every timed step recorded as HIP graphs (the calls before the dominant GEMM "
                         "launch, that launch, the calls after it) and timed as their replays; stream: the library "
                         "calls issued on the stream step by step; auto (default): graph for the two-launch "
                         "schedule, stream for the single launch")
    ap.add_argument("--block-m", type=int, default=0,
                    help="routing block rows to use instead of the workload's own (16, 32, 64 or 128)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="number of tokens to use instead of the workload's own (same routing recipe)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain elementwise copy (y = -x, float32) of this many MiB five times: the "
                         "reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.event_every < 1:
        print("bench.py: --event-every must be at least 1", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py: the library runs one GPU's share of the MoE layer; --gpus {args.gpus} is not supported "
              f"(no sharding across GPUs, no collectives)", file=sys.stderr)
        return 2

    import torch
    from moe_expert_ffn_plan_amd import binding as B
    from moe_expert_ffn_plan_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "dispatches": 5}), flush=True)
        return 0
    w = inputs.WORKLOADS[args.workload]
    if args.block_m:
        w = dataclasses.replace(w, block_m=args.block_m)
    if args.tokens:
        w = dataclasses.replace(w, num_tokens=args.tokens)
    if args.block_m or args.tokens:  # a different workload: no committed profile describes it
        w = dataclasses.replace(w, name=f"{w.name}_T{w.num_tokens}_bm{w.block_m}")
    s = B.shape_of(w)
    gen_dev = "cpu" if args.host_inputs else dev
    d = {k: v.to(dev) for k, v in inputs.make_inputs(w, device=gen_dev).items()}
    # one-time weight re-layout (untimed, like the pages' weight transform)
    weights = [B.prepare_all(s, d)]
    for c in range(1, args.weight_copies):
        wc = inputs.make_weights(w, device=gen_dev, weight_seed=w.weight_seed + 1000 * c)
        weights.append(B.prepare_all(s, {k: v.to(dev) for k, v in wc.items()}))
        del wc
    torch.cuda.synchronize()
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=dev)
    ws = torch.empty(B.forward_workspace_bytes(s), dtype=torch.uint8, device=dev)
    y = torch.empty(w.num_tokens, w.hidden, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    dev_ev = DeviceEvents()
    # the schedule moe_forward picks (moe_gemm_launches): one persistent launch for both GEMMs while
    # Linear1 has few tiles per CU, else the two GEMM launches
    fused = B.forward_uses_expert_ffn(s) and B.expert_ffn_is_fused(s) and not args.staged
    if args.expert_ffn:
        fused = B.expert_ffn_is_fused(s)
    # graph replay saves ~16 us per kernel boundary on the millisecond steps of the two-launch schedule;
    # on the sub-millisecond single-launch steps its three graph launches cost more than that (measured)
    launch = args.launch if args.launch != "auto" else ("stream" if fused or args.forward else "graph")

    def bind_calls(wt, staged):
        """The step's library calls in order, as (stage name, call on a stream), their arguments checked
        and marshalled once here (binding.Bound), so that the timed loop only enqueues; the dominant GEMM
        launch is the one named linear1 or expert_ffn."""
        if args.forward:
            return [("forward", B.forward(s, d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], wt["w1"], wt["w1_sf"],
                                          wt["w2"], wt["w2_sf"], y, ws, bind=True))]
        c = [("plan", B.plan(s, d["topk_idx"], plan_ws, bind=True))]
        if staged:
            c.append(("linear1", B.linear1(s, d["x"], d["x_sf"], d["topk_w"], wt["w1"], wt["w1_sf"], plan_ws, ws,
                                           bind=True)))
            c.append(("linear2", B.linear2(s, wt["w2"], wt["w2_sf"], plan_ws, ws, bind=True)))
        else:
            c.append(("expert_ffn", B.expert_ffn(s, d["x"], d["x_sf"], d["topk_w"], wt["w1"], wt["w1_sf"], wt["w2"],
                                                 wt["w2_sf"], plan_ws, ws, bind=True)))
        c.append(("combine", B.combine(s, plan_ws, ws, y, bind=True)))
        return c

    bound = {(c, staged): bind_calls(weights[c], staged) for c in range(len(weights)) for staged in (False, True)}

    def calls(i, staged):
        return bound[(i % len(weights), staged)]

    def step(i, events=None, k_events=None, staged=not fused):
        """One step; events: one per stage boundary; k_events: around the dominant GEMM launch."""
        stream = torch.cuda.current_stream()
        c = calls(i, staged)
        for j, (name, call) in enumerate(c):
            if events is not None:
                dev_ev.record(events[j], stream)
            dominant = k_events is not None and name in ("linear1", "expert_ffn", "forward")
            if dominant:
                dev_ev.record(k_events[0], stream)
            call(stream)
            if dominant:
                dev_ev.record(k_events[1], stream)
        if events is not None:
            dev_ev.record(events[len(c)], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    pv = B.plan_view(s, B.forward_view(s, ws)["plan_ws"] if args.forward else plan_ws)
    scal = pv["scalars"].cpu().tolist()
    r_pad, n_valid = scal[0], scal[2]
    touched = int((pv["counts"] > 0).sum().item())  # experts with at least one row
    ids = d["topk_idx"]
    hit_tokens = int(((ids >= 0) & (ids < w.num_experts)).any(dim=1).sum().item())

    # the workspace's status word reports a single-launch GEMM that gave up waiting (y is then NaN)
    status = B.forward_view(s, ws)["sync_status"]

    def check_status(what):
        torch.cuda.synchronize()
        if int(status.item()) != 0 or not bool(torch.isfinite(y.float()).all()):
            raise RuntimeError(f"bench.py: {what}: a GEMM launch gave up waiting or y is not finite")
    check_status("warmup")

    # timed steps: wall time; HIP events bracket only the dominant GEMM launch (same stream)
    # events around the dominant launch of every event_every-th timed step (each pair of records costs
    # the stream a few microseconds, which matters on the 0.1 ms steps)
    k_evs = [[dev_ev.new() for _ in range(2)] if i % args.event_every == 0 else None for i in range(args.steps)]
    if launch == "graph":
        # every timed step as three recorded graphs (the calls before the dominant GEMM launch, that
        # launch, the calls after it; the weight copies in turn): the events around the dominant launch
        # are recorded between the replays, on the stream they replay on.  Each graph is replayed once
        # untimed first.
        side = torch.cuda.Stream()
        segs = []
        for i in range(args.steps):
            c = calls(i, not fused)
            k = next(j for j, (name, _) in enumerate(c) if name in ("linear1", "expert_ffn", "forward"))
            parts = []
            for part in (c[:k], c[k:k + 1], c[k + 1:]):
                g = None
                if part:  # (the whole-forward call has nothing before or after it)
                    side.wait_stream(torch.cuda.current_stream())
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        for _, call in part:
                            call(torch.cuda.current_stream())
                parts.append(g)
            segs.append(parts)
        torch.cuda.synchronize()
        for parts in segs:
            for g in parts:
                if g is not None:
                    g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i, (pre, dom, post) in enumerate(segs):
            if pre is not None:
                pre.replay()
            if k_evs[i] is not None:
                dev_ev.record(k_evs[i][0], stream)
            dom.replay()
            if k_evs[i] is not None:
                dev_ev.record(k_evs[i][1], stream)
            if post is not None:
                post.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, k_events=k_evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    timed_evs = [e for e in k_evs if e is not None]
    k_ms = sum(dev_ev.elapsed_ms(e[0], e[1]) for e in timed_evs) / len(timed_evs)
    check_status("timed steps")

    # untimed breakdown passes: an event between every stage (and the two-launch path for comparison)
    def breakdown(staged):
        names = [name for name, _ in calls(0, staged)]
        evs = [[dev_ev.new() for _ in range(len(names) + 1)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(i, evs[i], staged=staged)
        torch.cuda.synchronize()
        return {name: sum(dev_ev.elapsed_ms(e[j], e[j + 1]) for e in evs) / args.steps
                for j, name in enumerate(names)}
    kern_ms = breakdown(not fused)
    staged_ms = breakdown(True) if fused and not args.forward else None

    H, I = w.hidden, w.intermediate
    useful = 2.0 * n_valid * 3 * H * I
    tflops = useful / (ms * 1e-3) / 1e12
    # GEMM M-tile: 128 rows (several routing blocks of one expert) from block_m 32 up, else one block
    bmg = 128 if w.block_m >= 32 else w.block_m
    # tile variant: 0 = M-tile of one routing block, 1 = several blocks of fewer rows, 2 = blocks of more
    tv = 0 if w.block_m == bmg else (1 if w.block_m < bmg else 2)
    epi = 0  # the fast SiLU epilogue without a clamp (the bench's default)
    if fused:
        k_flops = useful
        # the events bracket moe_expert_ffn: its one-thread prepare kernel (launch counter, status word)
        # and the single launch
        kname = (f"Linear1 + Linear2 in one launch (fused_prepare_kernel + gemm_fused_kernel<{bmg}, {tv}, "
                 f"{epi}>)")
    else:
        k_flops = 2.0 * n_valid * 2 * I * H
        kname = "Linear1 grouped GEMM (%s<%d, true, %d, %d>)" % (
            "gemm_pp_kernel" if (2 * I) % 512 == 0 else "gemm4_kernel", bmg, tv, epi)
    k_bytes = kernel_bytes(w, fused, n_valid, touched, hit_tokens)
    # whole step, compulsory: touched weights and scales, x and x_sf of tokens with a local hit, the
    # top-k ids and weights, y
    step_bytes = int(touched * 3 * I * H * (1 / 2 + 1 / 32) + hit_tokens * H * (1 + 1 / 32) +
                     w.num_tokens * w.topk * 12 + w.num_tokens * H * 2)
    if args.forward:  # the events bracket the whole forward: its roofline is the step's
        k_flops, k_bytes = useful, step_bytes
        kname = ("whole moe_forward (routing, " + ("single GEMM launch" if fused else "two GEMM launches") +
                 ", combine)")
    # the roofline that bounds the kernel: the larger of its MFMA time and its HBM time at peak
    if k_bytes / (PEAK_HBM_GBS * 1e9) > k_flops / (PEAK_MFMA_TFLOPS * 1e12):
        achieved, peak, unit, bound = k_bytes / (k_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = k_flops / (k_ms * 1e-3) / 1e12, PEAK_MFMA_TFLOPS, "TFLOP/s", "mfma"
    roofline = {"kernel": kname, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "algorithmic_flops": k_flops, "algorithmic_bytes": k_bytes,
                "traffic": None if args.forward else kernel_traffic("expert_ffn" if fused else "linear1", w.name)}
    out = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8e4m3 x fp4e2m1 (fp32 accumulate)", "data": "synthetic",
           "config": {"workload": w.name, "tokens": w.num_tokens, "hidden": H, "intermediate": I,
                      "local_experts": w.num_experts, "topk": w.topk, "block_m": w.block_m,
                      "valid_rows": n_valid, "padded_rows": r_pad, "weight_copies": args.weight_copies,
                      "launch": launch, "calls": "moe_forward" if args.forward else "stages"},
           "tokens_per_s": round(w.num_tokens / (ms * 1e-3), 1),
           "pct_of_mfma_peak": round(100 * tflops / PEAK_MFMA_TFLOPS, 2),
           "pct_of_hbm_peak": round(100 * step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
           "step_algorithmic_bytes": step_bytes,
           "gemm_ms": round(k_ms, 4),
           "kernel_ms": {k: round(v, 4) for k, v in kern_ms.items()},
           "roofline": roofline}
    if staged_ms is not None:
        out["staged_kernel_ms"] = {k: round(v, 4) for k, v in staged_ms.items()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, d, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
