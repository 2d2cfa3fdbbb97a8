#!/usr/bin/env python3
"""Benchmark: one step of the bucketed gradient sync on the GPT-2-small
gradient set, p = 8 simulated ranks in one GPU's HBM.

A step is one pass of the whole path over every bucket of the plan:
flatten (copy each rank's gradients into the bucket), ring all-reduce of the
bucket averaged over p (fused single-pass kernel), unflatten (copy back).
The plan is built once, before timing, as the reducer does at construction.

Printed: one JSON line with the all-reduce bus bandwidth of the whole step
(busBW = S * 2(p-1)/p / t_step, S = bytes of gradient per rank), the
roofline of the dominant kernel (the fused all-reduce) measured with HIP
events on the stream it runs on, and the CPU oracle timed on a bounded
sample of the same workload.

Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-buckets", type=int, default=0,
                    help="buckets in the CPU-baseline sample (0 = auto)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB "
                         "(for scaling hardware counters)")
    ap.add_argument("--algo", default="fused", choices=["fused", "ring"])
    return ap.parse_args()


def build_workload(torch, ddp, W, dev):
    cfg = W.WORKLOADS["gpt2-small-p8"]
    p = cfg["p"]
    params = cfg["params"]
    sizes = [W.numel(s) for _, s in params]
    plan = ddp.ddp_bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    plan.upload(dev)
    # one arena per rank, parameters in registration order at 256-byte
    # aligned offsets (as separate allocations would be)
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 63) // 64 * 64
    arenas, grads = [], []
    for r in range(p):
        a = torch.empty(off, dtype=torch.float32, device=dev)
        W.normal_torch(off, cfg["sigma"], cfg["seed"], r, dev, out=a)
        arenas.append(a)
        grads.append([a[o:o + n] for o, n in zip(offs, sizes)])
    table = ddp.grad_pointer_table(grads, dev)
    buckets = []
    for b in range(plan.num_buckets):
        nb = plan.bucket_numel(b)
        buckets.append([torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(p)])
    return cfg, p, sizes, plan, grads, table, buckets, arenas


def cpu_baseline(W, cfg, sizes, n_buckets_wanted):
    """The oracle (single thread) on the first buckets of the same plan:
    flatten, literal ring all-reduce averaged by p, unflatten."""
    import numpy as np
    import oracle

    p = cfg["p"]
    oplan = oracle.bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    nb = n_buckets_wanted or 4
    params = [i for b in range(nb) for i in oplan.bucket_params(b)]
    host = [[None] * len(sizes) for _ in range(p)]
    for r in range(p):
        for i in params:
            host[r][i] = W.normal_np(sizes[i], cfg["sigma"], cfg["seed"], r, stream=i)
    elems = sum(oplan.bucket_numel(b) for b in range(nb))
    t0 = time.perf_counter()
    for b in range(nb):
        flats = [oracle.flatten(host[r], oplan, b) for r in range(p)]
        red, _ = oracle.ring_allreduce(flats, avg="world", want_log=False)
        for r in range(p):
            oracle.unflatten(red[r], oplan, b, host[r])
    dt = time.perf_counter() - t0
    S = elems * 4
    bus = S * 2 * (p - 1) / p / dt / 1e9
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(bus, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"first {nb} of {oplan.num_buckets} buckets ({elems} fp32 elements "
                   f"per rank, p={p}): flatten + literal ring all-reduce (avg by p) + "
                   f"unflatten, single thread, {dt:.2f} s on {cpu}"),
        "seconds": round(dt, 3),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the p ranks are simulated inside one GPU's "
              "HBM, so there is nothing to run on more than one GPU.", file=sys.stderr)
        sys.exit(2)
    import torch

    import bucketed_gradient_all_ddp_amd as ddp
    from bucketed_gradient_all_ddp_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    ddp.load_library()
    log("building workload")
    cfg, p, sizes, plan, grads, table, buckets, arenas = build_workload(torch, ddp, W, dev)
    S = sum(sizes) * 4
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ws = {}
    if args.algo == "ring":
        for b in range(plan.num_buckets):
            need = ddp.ring_allreduce_sim_workspace(p, plan.bucket_numel(b), 0, "ring")
            ws[b] = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None

    def step(events=None):
        for b in range(plan.num_buckets):
            bufs = buckets[b]
            ddp.ddp_flatten(plan, b, table, bufs)
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            st = ddp.ring_allreduce_sim(bufs, avg="world", algo=args.algo,
                                        workspace=ws.get(b))
            if events is not None:
                e1.record(stream)
                events.append((st.hbm_bytes, e0, e1))
            ddp.ddp_unflatten(plan, b, bufs, table)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps

    # the dominant kernel (fused all-reduce), timed per launch with events on
    # the stream it is launched on
    events = []
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    ar_ms = sum(e0.elapsed_time(e1) for _, e0, e1 in events)
    ar_launches = len(events)
    ar_bytes = sum(hbm for hbm, _, _ in events)
    achieved = ar_bytes / (ar_ms * 1e-3) / 1e9
    ar_per_step_ms = ar_ms / args.steps
    log(f"step {ms:.3f} ms, all-reduce {ar_per_step_ms:.3f} ms/step "
        f"({ar_launches // args.steps} launches), {achieved:.0f} GB/s algorithmic")

    calib = None
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 1024 * 1024 // 4
        a = torch.empty(n, device=dev)
        b2 = torch.empty(n, device=dev)
        a.fill_(1.0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            b2.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / reps
        calib = {"bytes": 2 * n * 4, "ms": round(cms, 4),
                 "GBps": round(2 * n * 4 / (cms * 1e-3) / 1e9, 1)}
        log(f"copy {args.calib_copy_mib} MiB: {calib}")

    bus = S * 2 * (p - 1) / p / (ms * 1e-3) / 1e9
    step_bytes = 6 * p * S  # flatten + all-reduce + unflatten, each 2pS
    result = {
        "metric": "all-reduce bus GB/s + % HBM peak, p=8 sim ranks, 124M fp32 grads",
        "value": round(bus, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "gpt2-small gradients (148 fp32 tensors, 124,439,808 elements "
                        "per rank), p=8 simulated ranks, 25 MiB buckets + 1 MiB first "
                        "bucket (13 buckets), average by p; step = flatten + "
                        f"{args.algo} ring all-reduce + unflatten per bucket",
            "p": p, "buckets": plan.num_buckets, "bytes_per_rank": S,
        },
        "hbm_frac_step": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "allreduce": {
            "ms_per_step": round(ar_per_step_ms, 4),
            "bus_GBps": round(S * 2 * (p - 1) / p / (ar_per_step_ms * 1e-3) / 1e9, 2),
            "launches_per_step": ar_launches // args.steps,
        },
        "roofline": {
            "kernel": "fused_allreduce_kernel" if args.algo == "fused" else "ring_step_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
    }
    if calib:
        result["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(W, cfg, sizes, args.cpu_buckets)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
