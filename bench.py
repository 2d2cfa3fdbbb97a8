#!/usr/bin/env python3
"""Benchmark: one bucketed gradient-sync step on the GPT-2-small gradient
set, p = 8 simulated ranks in one GPU's HBM.

A step is one pass of the whole path over every bucket of the plan: the
bucket's flatten, ring all-reduce averaged over p, and unflatten back into
each rank's per-parameter gradients. With no backward pass in the step,
every bucket is ready at once, and the reducer's rule -- launch the next
bucket and every following complete one -- makes them one run: the headline
("batched") step does flatten + all-reduce + unflatten in place for that
run in one kernel launch (ddp_allreduce_buckets; each bucket keeps its own
ring chunks, same bits as one launch per bucket). "inplace" launches that
kernel once per bucket (ddp_allreduce_bucket); "copy" runs the three steps
as three kernels per bucket (ddp_flatten, ring_allreduce_sim,
ddp_unflatten). All three are timed and reported. The plan is built once before timing, as the reducer
does at construction.

Output: one JSON line. `value` is the all-reduce bus bandwidth of the whole
step, S * 2(p-1)/p / t_step (S = gradient bytes per rank). `roofline` is for
the dominant kernel: its algorithmic bytes per launch over its launch
durations, measured with HIP events attached to the kernel dispatches on the
stream they run on, inside the timed region. `cpu_baseline` times the CPU
oracle (one thread) on the same workload.

One GPU only: --gpus above 1 is refused.
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
METRIC = "all-reduce bus GB/s + % HBM peak, p=8 sim ranks, 124M fp32 grads"

# Device-memory traffic per launch of a kernel: the DRAM-side request counters
# of a rocprofv3 --pmc pass (TCC_EA0_RDREQ_DRAM_32B_sum and
# TCC_EA0_WRREQ_WRITE_DRAM_32B_sum, 32-byte units, read + write), which read
# back a plain 1 GiB copy exactly (no scale factor), summarised in profiles/.
# A figure is used only while the kernel's sources hash to the value it was
# measured with; after any change it is reported as null until the counters
# are taken again.
CSRC = os.path.join(ROOT, "bucketed_gradient_all_ddp_amd", "csrc")
KERNEL_SOURCES = {
    # the kernel, the headers it includes, and the host code that shapes its
    # launch (residency bound) and builds the descriptor table and tile map it reads
    "bucket_allreduce_kernel": ["bucket_allreduce.hip", "fold.hpp", "internal.hpp",
                                "host.cpp", "plan.cpp"],
    "fused_allreduce_kernel": ["allreduce.hip", "fold.hpp", "internal.hpp", "host.cpp"],
}
MEASURED_TRAFFIC = {
    # profiles/bucket_allreduce_gpt2_p8.md: the headline launch (all 13
    # buckets in one dispatch), 3,984,249,536 read + 3,982,158,746 written
    "bucket_allreduce_kernel": {
        "bytes_per_launch": 7966408282,
        "sources_sha256": "76ddd334aeba600aefb1aa94f7f9a85a567df5f46f89a254e6932a37598151b8",
    },
}


def sources_sha256(kernel: str):
    import hashlib

    files = KERNEL_SOURCES.get(kernel)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    m = MEASURED_TRAFFIC.get(kernel)
    if m is None or m["sources_sha256"] != sources_sha256(kernel):
        return None
    return m["bytes_per_launch"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", default="batched", choices=["batched", "inplace", "copy"],
                    help="headline step: one launch for the run of all ready "
                         "buckets (ddp_allreduce_buckets), one launch per bucket "
                         "(ddp_allreduce_bucket), or flatten + all-reduce + "
                         "unflatten as three launches per bucket")
    ap.add_argument("--algo", default="fused", choices=["fused", "ring"],
                    help="all-reduce algorithm of the copy step")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the other step mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-buckets", type=int, default=0,
                    help="buckets in the CPU-baseline sample (0 = all)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also time a plain device copy of this many MiB")
    ap.add_argument("--workload", default="gpt2-small-p8",
                    choices=["gpt2-small-p8", "ragged-ring-p4", "llama7b-bf16-p8",
                             "latency-p64", "cost-model-p64", "overlap-gpt2-p8",
                             "crossover-p4", "sync-gpt2-p8", "collectives-p8", "ceilings"],
                    help="the default is the headline; the others print their own "
                         "line for the record")
    ap.add_argument("--tokens", type=int, default=2048,
                    help="tokens per synthetic backward GEMM (overlap workload)")
    ap.add_argument("--no-per-tensor-loop", action="store_true",
                    help="latency workload: skip the 20,000 per-tensor launches (loop and "
                         "graph replay), e.g. under a counter profiler")
    ap.add_argument("--comm-workgroups", type=str, default="0,256,1024,4096",
                    help="overlap workload: caps on the reducer's all-reduce workgroups "
                         "to time (0 = one per tile)")
    return ap.parse_args()


class Workload:
    def __init__(self, torch, ddp, W, dev):
        cfg = W.WORKLOADS["gpt2-small-p8"]
        self.cfg = cfg
        self.p = p = cfg["p"]
        self.sizes = sizes = [W.numel(s) for _, s in cfg["params"]]
        self.S = sum(sizes) * 4
        plan = ddp.ddp_bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
        plan.upload(dev)
        plan.upload_segments(p, dev)
        self.plan = plan
        self.nb = [plan.bucket_numel(b) for b in range(plan.num_buckets)]
        # one arena per rank, parameters in registration order at 256-byte
        # aligned offsets (as separate allocations would be)
        offs, off = [], 0
        for n in sizes:
            offs.append(off)
            off += (n + 63) // 64 * 64
        self.arenas, grads = [], []
        for r in range(p):
            a = torch.empty(off, dtype=torch.float32, device=dev)
            W.normal_torch(off, cfg["sigma"], cfg["seed"], r, dev, out=a)
            self.arenas.append(a)
            grads.append([a[o:o + n] for o, n in zip(offs, sizes)])
        self.offs = offs
        self.grads = grads
        self.host_arenas = None
        self.table = ddp.grad_pointer_table(grads, dev)
        self.buckets = None

    def ensure_bucket_buffers(self, torch, dev):
        if self.buckets is None:
            self.buckets = [[torch.empty(n, dtype=torch.float32, device=dev)
                             for _ in range(self.p)] for n in self.nb]


def run_steps(ddp, wl, mode, algo, steps, timer, ws):
    """Run `steps` steps; when a timer is given, every kernel call is timed
    by events attached to its dispatches. Returns [(kind, bytes, id)]."""
    rec = []
    plan, p, table = wl.plan, wl.p, wl.table
    for _ in range(steps):
        if mode == "batched":
            k = timer.arm() if timer else None
            st = ddp.ddp_allreduce_buckets(plan, 0, plan.num_buckets, table, p, avg="world")
            if timer:
                rec.append(("bucket_allreduce_kernel", st.hbm_bytes, k))
            continue
        for b in range(plan.num_buckets):
            if mode == "inplace":
                k = timer.arm() if timer else None
                st = ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
                if timer:
                    rec.append(("bucket_allreduce_kernel", st.hbm_bytes, k))
            else:
                bufs = wl.buckets[b]
                k = timer.arm() if timer else None
                ddp.ddp_flatten(plan, b, table, bufs)
                if timer:
                    rec.append(("flatten_kernel", 2 * p * wl.nb[b] * 4, k))
                k = timer.arm() if timer else None
                st = ddp.ring_allreduce_sim(bufs, avg="world", algo=algo, workspace=ws.get(b))
                if timer:
                    rec.append(("fused_allreduce_kernel" if algo == "fused" else "ring_step_kernel",
                                st.hbm_bytes, k))
                k = timer.arm() if timer else None
                ddp.ddp_unflatten(plan, b, bufs, table)
                if timer:
                    rec.append(("unflatten_kernel", 2 * p * wl.nb[b] * 4, k))
    return rec


def timed(torch, ddp, wl, mode, algo, steps, warmup, ws):
    """(ms per step, per-kernel figures, ms per step with the kernel events).

    The step time comes from a pass with no per-call events: recording a
    start and a stop event on every dispatch costs about 5 us of GPU time per
    launch (13 launches per step in the per-bucket form). A second pass of
    the same steps times every kernel by events on its own dispatch."""
    run_steps(ddp, wl, mode, algo, warmup, None, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(ddp, wl, mode, algo, steps, None, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    per_step_calls = {"batched": 1, "inplace": wl.plan.num_buckets,
                      "copy": 3 * wl.plan.num_buckets}[mode]
    timer = ddp.CallTimer(pairs=per_step_calls * steps)
    t0 = time.perf_counter()
    rec = run_steps(ddp, wl, mode, algo, steps, timer, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_events = (t1 - t0) * 1e3 / steps
    kernels = {}
    for kind, nbytes, k in rec:
        e = kernels.setdefault(kind, {"launches": 0, "bytes": 0, "ms": 0.0})
        e["launches"] += 1
        e["bytes"] += nbytes
        e["ms"] += timer.elapsed_ms(k)
    for e in kernels.values():
        e["avg_us"] = round(1e3 * e["ms"] / e["launches"], 2)
        e["GBps"] = round(e["bytes"] / (e["ms"] * 1e-3) / 1e9, 1)
        e["ms_per_step"] = round(e["ms"] / steps, 4)
        e["ms"] = round(e["ms"], 4)
    return ms, kernels, ms_events


def _host_cpu() -> str:
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return cpu


def cpu_record(value, unit, sample, seconds=None):
    """A cpu_baseline object: the oracle runs on one thread ("cores"); the
    host's core count and model are stated beside it."""
    rec = {"value": value, "unit": unit, "cores": 1, "kind": "oracle", "sample": sample,
           "host_cores": os.cpu_count(), "host_cpu": _host_cpu()}
    try:
        rec["host_cores_usable"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    if seconds is not None:
        rec["seconds"] = round(seconds, 3)
    return rec


def host_copy(t):
    """A device tensor's values on the host (bf16 as uint16 bit patterns),
    for the oracle."""
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view("uint16")
    return t.cpu().numpy()


def cpu_oracle_ring(bufs, avg="world", tokens=None, what=""):
    """The oracle's literal ring all-reduce on host arrays, one thread: the
    CPU-baseline leg of the non-headline workloads. Returns (seconds, the
    cpu_baseline object's text)."""
    import oracle

    t0 = time.perf_counter()
    oracle.ring_allreduce(bufs, avg=avg, tokens=tokens, want_log=False)
    dt = time.perf_counter() - t0
    return dt, f"{what}: literal ring all-reduce, one thread, {dt:.2f} s on {_host_cpu()}"


def cpu_baseline(W, wl, n_buckets_wanted):
    """The oracle (single thread): flatten, literal ring all-reduce averaged
    by p, unflatten, over the first buckets of the same plan, on the values
    the GPU started from (read back before any kernel ran)."""
    import oracle

    p, sizes = wl.p, wl.sizes
    oplan = oracle.bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    nb = n_buckets_wanted or oplan.num_buckets
    host = [[a[o:o + n] for o, n in zip(wl.offs, sizes)] for a in wl.host_arenas]
    elems = sum(oplan.bucket_numel(b) for b in range(nb))
    t0 = time.perf_counter()
    for b in range(nb):
        flats = [oracle.flatten(host[r], oplan, b) for r in range(p)]
        red, _ = oracle.ring_allreduce(flats, avg="world", want_log=False)
        for r in range(p):
            oracle.unflatten(red[r], oplan, b, host[r])
    dt = time.perf_counter() - t0
    S = elems * 4
    return cpu_record(
        round(S * 2 * (p - 1) / p / dt / 1e9, 4), "GB/s",
        f"{nb} of {oplan.num_buckets} buckets ({elems} fp32 elements per rank, p={p}, the "
        f"GPU's own input values read back before its first kernel): flatten + literal ring "
        f"all-reduce (avg by p) + unflatten, one thread, {dt:.2f} s", dt)


# ---------------------------------------------------------------------------
# Other workloads (not the headline): one JSON line each
# ---------------------------------------------------------------------------

def _events_ms(torch, fn, reps):
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _timed_calls(torch, ddp, calls, reps, wall=True):
    """Each call once per rep. Returns (host wall ms per rep, device ms per
    rep). The wall time comes from a pass without events (an event pair on
    every dispatch costs about 5 us of GPU time per launch); a second pass
    times every call's kernels by events on their own dispatches. wall=False
    skips the first pass (and returns None for it)."""
    wall_ms = None
    if wall:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            for c in calls:
                c()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / reps
    timer = ddp.CallTimer(pairs=len(calls) * reps)
    ids = []
    torch.cuda.synchronize()
    for _ in range(reps):
        for c in calls:
            ids.append(timer.arm())
            c()
    torch.cuda.synchronize()
    dev = sum(timer.elapsed_ms(k) for k in ids) / reps
    return wall_ms, dev


def _line(metric, value, unit, workload, extra):
    d = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1,
         "higher_is_better": True, "data": "synthetic", "config": {"workload": workload}}
    d.update(extra)
    print(json.dumps(d), flush=True)


def bench_ragged(torch, ddp, W, dev, args):
    cfg = W.WORKLOADS["ragged-ring-p4"]
    p, n = cfg["p"], cfg["n"]
    bufs = [W.normal_torch(n, 1.0, cfg["seed"], r, dev) for r in range(p)]
    host = [host_copy(b) for b in bufs]
    out = {}
    for algo in ("fused", "ring"):
        for _ in range(args.warmup):
            ddp.ring_allreduce_sim(bufs, avg="world", algo=algo)
        wall, dms = _timed_calls(torch, ddp, [lambda: ddp.ring_allreduce_sim(
            bufs, avg="world", algo=algo)], args.steps)
        S = n * 4
        st = ddp.ring_allreduce_sim(bufs, avg="world", algo=algo)
        out[algo] = {"device_us": round(dms * 1e3, 2), "wall_us": round(wall * 1e3, 2),
                     "bus_GBps": round(S * 2 * (p - 1) / p / (dms * 1e-3) / 1e9, 1),
                     "hbm_GBps": round(st.hbm_bytes / (dms * 1e-3) / 1e9, 1),
                     "launches": 1 if algo == "fused" else 2 * (p - 1)}
    extra = {"algorithms": out}
    if not args.no_cpu_baseline:
        dt, text = cpu_oracle_ring(host, "world", None,
                                   f"the whole workload (p={p}, n={n}, the GPU's input values)")
        extra["cpu_baseline"] = cpu_record(round(n * 4 * 2 * (p - 1) / p / dt / 1e9, 4),
                                           "GB/s", text, dt)
    _line("all-reduce bus GB/s, p=4, 1,000,003 fp32 per rank", out["fused"]["bus_GBps"], "GB/s",
          "ragged ring: one 1,000,003-element fp32 tensor per rank, p=4, average by p", extra)


def bench_llama(torch, ddp, W, dev, args):
    cfg = W.WORKLOADS["llama7b-bf16-p8"]
    p = cfg["p"]
    sizes = [W.numel(s) for _, s in cfg["params"]]
    plan = ddp.ddp_bucket_plan(sizes, 2, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    plan.upload_segments(p, dev)
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 127) // 128 * 128
    arenas = []
    for r in range(p):
        a = torch.empty(off, dtype=torch.bfloat16, device=dev)
        piece = 1 << 28
        for k, lo in enumerate(range(0, off, piece)):
            hi = min(off, lo + piece)
            a[lo:hi].copy_(W.normal_torch(hi - lo, cfg["sigma"], cfg["seed"], r, dev, stream=k))
        arenas.append(a)
    grads = [[a[o:o + n] for o, n in zip(offs, sizes)] for a in arenas]
    table = ddp.grad_pointer_table(grads, dev)
    # the oracle's sample: bucket 1's gradients as the GPU starts from them
    cpu_in = None
    if not args.no_cpu_baseline:
        cpu_in = [{i: host_copy(grads[r][i]) for i in plan.bucket_params(1)} for r in range(p)]
    calls = [lambda b=b: ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
             for b in range(plan.num_buckets)]
    for _ in range(max(1, args.warmup // 2)):
        for c in calls:
            c()
    reps = max(2, args.steps // 4)
    wall, dms = _timed_calls(torch, ddp, calls, reps)
    S = sum(sizes) * 2
    hbm = 2 * p * S
    # every bucket ready at once: one launch for the whole run
    nb = plan.num_buckets
    batched = [lambda: ddp.ddp_allreduce_buckets(plan, 0, nb, table, p, avg="world")]
    batched[0]()
    bwall, bdms = _timed_calls(torch, ddp, batched, reps)
    _line("all-reduce bus GB/s, p=8, Llama-7B bf16 grads", S * 2 * (p - 1) / p / (wall * 1e-3) / 1e9,
          "GB/s", "llama-7b gradients: 291 bf16 tensors, 6,738,415,616 elements per rank, p=8, "
                  "226 buckets (25 MiB / 1 MiB), fp32 accumulation, average by p; step = one "
                  "ddp_allreduce_bucket per bucket",
          {"ms_per_step": round(wall, 3), "kernel_ms_per_step": round(dms, 3),
           "kernel_GBps": round(hbm / (dms * 1e-3) / 1e9, 1),
           "kernel_frac_of_8TBps": round(hbm / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "one_launch_for_all_buckets": {
               "ms_per_step": round(bwall, 3), "kernel_ms_per_step": round(bdms, 3),
               "bus_GBps": round(S * 2 * (p - 1) / p / (bwall * 1e-3) / 1e9, 1),
               "kernel_GBps": round(hbm / (bdms * 1e-3) / 1e9, 1),
               "kernel_frac_of_8TBps": round(hbm / (bdms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
           "dtype": "bf16 (fp32 accumulate)", "steps": reps,
           **({} if args.no_cpu_baseline else {"cpu_baseline": _llama_cpu(W, sizes, p, cpu_in)})})


def _llama_cpu(W, sizes, p, cpu_in):
    """Oracle on a sample of the Llama-7B buckets (the whole set does not fit
    a host comfortably): bucket 1 of the plan (one 4096 x 11008 tensor), on
    the GPU's own bf16 input values: flatten, ring all-reduce in fp32,
    unflatten."""
    import oracle

    oplan = oracle.bucket_plan(sizes, 2, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    b = 1
    n = oplan.bucket_numel(b)
    host = [[cpu_in[r].get(i) for i in range(len(sizes))] for r in range(p)]
    t0 = time.perf_counter()
    flats = [oracle.flatten(host[r], oplan, b) for r in range(p)]
    red, _ = oracle.ring_allreduce(flats, avg="world", want_log=False)
    for r in range(p):
        oracle.unflatten(red[r], oplan, b, host[r])
    dt = time.perf_counter() - t0
    return cpu_record(
        round(n * 2 * 2 * (p - 1) / p / dt / 1e9, 4), "GB/s",
        f"bucket 1 of {oplan.num_buckets} ({n} bf16 elements per rank, p={p}, the GPU's own "
        f"input values): flatten + literal ring all-reduce in fp32 + unflatten, one thread, "
        f"{dt:.2f} s", dt)


def bench_latency(torch, ddp, W, dev, args):
    cfg = W.WORKLOADS["latency-p64"]
    p, sizes = cfg["p"], cfg["sizes"]
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 63) // 64 * 64
    arenas = [W.normal_torch(off, 1.0, cfg["seed"], r, dev) for r in range(p)]
    grads = [[a[o:o + n] for o, n in zip(offs, sizes)] for a in arenas]
    per_tensor = [[grads[r][i] for r in range(p)] for i in range(len(sizes))]
    S = sum(sizes) * 4
    hbm = 2 * p * S
    # the oracle's sample: the first tensors as the GPU starts from them
    cpu_in = None if args.no_cpu_baseline else [
        [host_copy(t) for t in per_tensor[i]] for i in range(min(1000, len(sizes)))]

    def tensor_step():
        for bufs in per_tensor:
            ddp.ring_allreduce_sim(bufs, avg="world")

    host_ms = graph_ms = float("nan")
    if not args.no_per_tensor_loop:
        tensor_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tensor_step()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3
        # the same 20,000 launches replayed from a captured HIP graph
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            tensor_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            tensor_step()
        g.replay()
        torch.cuda.synchronize()
        graph_ms = _events_ms(torch, g.replay, 3)
        del g
    plan = ddp.ddp_bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    plan.upload_segments(p, dev)
    table = ddp.grad_pointer_table(grads, dev)
    calls = [lambda b=b: ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
             for b in range(plan.num_buckets)]
    for c in calls:
        c()
    wall, dms = _timed_calls(torch, ddp, calls, 5)
    nb = plan.num_buckets
    one = [lambda: ddp.ddp_allreduce_buckets(plan, 0, nb, table, p, avg="world")]
    one[0]()
    owall, odms = _timed_calls(torch, ddp, one, 5)
    # the per-tensor arithmetic (every tensor padded and chunked on its own)
    # in one launch: caps of 0 bytes give every tensor a bucket of its own
    tplan = ddp.ddp_bucket_plan(sizes, 4, 0, 0)
    tplan.upload_segments(p, dev)
    tone = [lambda: ddp.ddp_allreduce_buckets(tplan, 0, tplan.num_buckets, table, p,
                                              avg="world")]
    tone[0]()
    twall, tdms = _timed_calls(torch, ddp, tone, 5)
    _line("all-reduce step time, p=64, 20,000 tensors: bucketed vs per-tensor",
          graph_ms / wall, "x (per-tensor graph time / bucketed time)",
          "latency regime: 20,000 fp32 tensors of 64..65,536 elements (189,015,250 per rank), "
          "p=64, average by p",
          {"per_tensor": {"launches": len(sizes), "host_loop_ms": round(host_ms, 2),
                          "graph_replay_ms": round(graph_ms, 2),
                          "graph_us_per_launch": round(graph_ms * 1e3 / len(sizes), 2),
                          "hbm_GBps_graph": round(hbm / (graph_ms * 1e-3) / 1e9, 1),
                          "one_launch_for_all_tensors": {
                              "ms_per_step": round(twall, 3),
                              "kernel_ms_per_step": round(tdms, 3),
                              "kernel_GBps": round(hbm / (tdms * 1e-3) / 1e9, 1)}},
           "bucketed": {"buckets": plan.num_buckets, "ms_per_step": round(wall, 3),
                        "kernel_ms_per_step": round(dms, 3),
                        "kernel_GBps": round(hbm / (dms * 1e-3) / 1e9, 1),
                        "one_launch_for_all_buckets": {
                            "ms_per_step": round(owall, 3), "kernel_ms_per_step": round(odms, 3),
                            "kernel_GBps": round(hbm / (odms * 1e-3) / 1e9, 1)}},
           **({} if args.no_cpu_baseline else {"cpu_baseline": _latency_cpu(sizes, p, cpu_in)})})


def _latency_cpu(sizes, p, cpu_in):
    """Oracle on the first of the 20,000 tensors (the GPU's own input
    values), one ring all-reduce per tensor (the per-tensor mode's
    arithmetic)."""
    total, elems = 0.0, 0
    for bufs in cpu_in:
        dt, _ = cpu_oracle_ring(bufs, "world")
        total += dt
        elems += bufs[0].size
    return cpu_record(
        round(elems * 4 * 2 * (p - 1) / p / total / 1e9, 4), "GB/s",
        f"the first {len(cpu_in)} of {len(sizes)} tensors ({elems} fp32 elements per rank, "
        f"p={p}, the GPU's own input values), one literal ring all-reduce each, one thread, "
        f"{total:.2f} s", total)


def bench_collectives_p8(torch, ddp, W, dev, args):
    bench_costmodel(torch, ddp, W, dev, args, "collectives-p8")


def bench_costmodel(torch, ddp, W, dev, args, name="cost-model-p64"):
    cfg = W.WORKLOADS[name]
    p, n = cfg["p"], cfg["n"]
    tokens = W.token_counts(p, cfg["seed"])
    bufs = [W.normal_torch(n, 1.0, cfg["seed"], r, dev) for r in range(p)]
    # the oracle's sample: one 8 MiB window of every rank, as the GPU starts
    cpu_in = None if args.no_cpu_baseline else [host_copy(b[:1 << 21]) for b in bufs]
    S = n * 4
    C = n // p
    outs = [torch.empty(C, device=dev) for _ in range(p)]
    shards = [bufs[r][r * C:(r + 1) * C] for r in range(p)]
    ops = {
        "allreduce_tokens": (lambda: ddp.ring_allreduce_sim(bufs, avg="tokens", tokens=tokens),
                             2 * (p - 1) / p, 2 * p * S),
        "reduce_scatter": (lambda: ddp.reduce_scatter_sim(bufs, outs), (p - 1) / p, (p + 1) * S),
        "allgather_inplace": (lambda: ddp.allgather_sim(shards, bufs), (p - 1) / p, p * S),
        "broadcast": (lambda: ddp.broadcast_sim(bufs, src=0), 1.0, p * S),
    }
    # the same all-reduce under the logarithmic schedules, fused (one pass each)
    for sch in ("recursive_doubling", "rabenseifner", "tree"):
        ops[f"allreduce_tokens_{sch}"] = (
            lambda s=sch: ddp.allreduce_sim(bufs, s, False, avg="tokens", tokens=tokens),
            2 * (p - 1) / p, 2 * p * S)
    # the ring schedule step by step: 2(p-1) launches, each a ring step
    # (reduce-scatter step: read sender and receiver, write receiver, 3n
    # elements; all-gather step: read sender, write receiver, 2n), averaged
    # by p so that repeated runs keep their magnitude
    ops["allreduce_ring_steps"] = (lambda: ddp.ring_allreduce_sim(bufs, avg="world",
                                                                  algo="ring"),
                                   2 * (p - 1) / p, 5 * (p - 1) * S)
    res = {}
    for name, (fn, busf, hbm) in ops.items():
        fn()
        wall, dms = _timed_calls(torch, ddp, [fn], 3)
        res[name] = {"device_ms": round(dms, 3), "alg_GBps": round(S / (dms * 1e-3) / 1e9, 1),
                     "bus_GBps": round(S * busf / (dms * 1e-3) / 1e9, 1),
                     "hbm_GBps": round(hbm / (dms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(hbm / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log(f"{name}: {res[name]['device_ms']} ms, {res[name]['hbm_GBps']} GB/s")
    # each ring step on its own (one launch per call, timed by its dispatch
    # events): reduce-scatter steps move 3n elements, all-gather steps 2n
    steps = [lambda k=k: ddp.ring_allreduce_sim_steps(bufs, k, 1, avg="world")
             for k in range(2 * (p - 1))]
    timer = ddp.CallTimer(pairs=len(steps) * 3)
    ids = []
    for _ in range(3):
        for k, fn in enumerate(steps):
            ids.append((k, timer.arm()))
            fn()
    torch.cuda.synchronize()
    per = {"reduce_scatter": [], "allgather": []}
    for k, i in ids:
        per["reduce_scatter" if k < p - 1 else "allgather"].append(timer.elapsed_ms(i))
    res["ring_step_kernel"] = {}
    for kind, elems in (("reduce_scatter", 3), ("allgather", 2)):
        us = 1e3 * sum(per[kind]) / len(per[kind])
        res["ring_step_kernel"][kind] = {
            "launches": len(per[kind]), "avg_us": round(us, 2),
            "bytes_per_launch": elems * S,
            "hbm_GBps": round(elems * S / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(elems * S / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    gib = n * 4 / (1 << 30)
    what = ("cost-model shape: one 2^29-element fp32 tensor per rank (2 GiB), p=64"
            if name == "cost-model-p64" else
            f"flat collectives: one 2^{n.bit_length() - 1}-element fp32 tensor per rank "
            f"({gib:g} GiB), p={p}")
    _line(f"all-reduce bus GB/s, p={p}, {gib:g} GiB fp32 per rank, token-weighted",
          res["allreduce_tokens"]["bus_GBps"], "GB/s",
          what + ", tokens U{10..10000}; plus reduce-scatter, in-place all-gather, "
          "broadcast, the all-reduce under recursive doubling, Rabenseifner and the "
          "tree (fused), and the ring step by step (2(p-1) launches, averaged by p)",
          {"ops": res, **({} if args.no_cpu_baseline else {"cpu_baseline": _costmodel_cpu(
              p, tokens, cpu_in)})})


def _costmodel_cpu(p, tokens, cpu_in):
    """Oracle on the first window of 2^21 elements (8 MiB) of every rank's
    tensor (the GPU's own input values), token-weighted: the full tensors do
    not fit a host comfortably."""
    window = cpu_in[0].size
    dt, text = cpu_oracle_ring(cpu_in, "tokens", tokens,
                               f"the first 8 MiB window of each rank's tensor (p={p}, the "
                               f"GPU's own input values)")
    return cpu_record(round(window * 4 * 2 * (p - 1) / p / dt / 1e9, 4), "GB/s", text, dt)


def bench_overlap(torch, ddp, W, dev, args):
    """Synthetic backward on one stream, bucket all-reduces on another,
    launched by the reducer as parameters are marked ready."""
    wl = Workload(torch, ddp, W, dev)
    p, sizes, plan = wl.p, wl.sizes, wl.plan
    params = wl.cfg["params"]
    # gradient values the "backward" writes: a copy of the drawn gradients
    sources = [a.clone() for a in wl.arenas]
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 63) // 64 * 64
    src_views = [[s_[o:o + n] for o, n in zip(offs, sizes)] for s_ in sources]
    # compute: per 2-D parameter (a, b) one bf16 GEMM [a, T] x [T, b], the
    # shape of a weight gradient over T tokens
    T = args.tokens
    gemms = {}
    for i, (_, shape) in enumerate(params):
        if len(shape) == 2:
            a, b = shape
            gemms[i] = (torch.randn(a, T, device=dev, dtype=torch.bfloat16),
                        torch.randn(T, b, device=dev, dtype=torch.bfloat16),
                        torch.empty(a, b, device=dev, dtype=torch.bfloat16))
    producer = torch.cuda.Stream()
    comm = torch.cuda.Stream()
    reducer = ddp.Reducer(plan, p, wl.table, avg="world", comm_stream=comm)
    order = list(range(len(sizes)))[::-1]
    events = [torch.cuda.Event() for _ in sizes]  # created once, re-recorded
    dsts = [[wl.grads[r][i] for r in range(p)] for i in range(len(sizes))]
    srcs = [[src_views[r][i] for r in range(p)] for i in range(len(sizes))]

    def backward(mark, clock=None):
        with torch.cuda.stream(producer):
            if clock is not None:
                clock[0].record(producer)
            for i in order:
                if i in gemms:
                    A, B, O = gemms[i]
                    torch.mm(A, B, out=O)
                torch._foreach_copy_(dsts[i], srcs[i])
                if clock is not None:
                    clock[1][i].record(producer)
                if mark:
                    events[i].record(producer)
                    reducer.mark_ready(i, events[i])

    def run(kind):
        cur = torch.cuda.current_stream()
        producer.wait_stream(cur)
        comm.wait_stream(cur)
        if kind == "overlap":
            reducer.prepare()
            backward(True)
            reducer.finalize(cur)
            cur.wait_stream(producer)
        else:
            backward(False)
            cur.wait_stream(producer)
            if kind == "sequential":
                for b in range(plan.num_buckets):
                    ddp.ddp_allreduce_bucket(plan, b, wl.table, p, avg="world")

    def timed_ms(kind):
        for _ in range(args.warmup):
            run(kind)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run(kind)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    res = {}
    for kind in ("backward_only", "sequential"):
        res[kind] = timed_ms(kind)
    capped = {}
    for cap in [int(c) for c in args.comm_workgroups.split(",")]:
        reducer.set_max_workgroups(cap)
        capped[cap] = timed_ms("overlap")
    best_cap = min(capped, key=capped.get)
    res["overlap"] = capped[best_cap]
    gemm_flops = sum(2 * T * W.numel(params[i][1]) for i in gemms)
    exposed_seq = res["sequential"] - res["backward_only"]
    exposed_ovl = res["overlap"] - res["backward_only"]
    model = _overlap_model(torch, ddp, plan, p, wl.table, backward, len(sizes))
    _line("exposed all-reduce time per step, overlapped vs after backward",
          exposed_ovl, "ms", "gpt2-small gradients, p=8: synthetic backward (per parameter "
          f"in reverse order: a bf16 GEMM [a,{T}]x[{T},b] for each 2-D parameter, then its "
          "gradients written for all ranks) on one stream; the reducer launches bucket "
          "all-reduces on a second stream as parameters are marked ready",
          {"higher_is_better": False,
           "ms_per_step": {k: round(v, 3) for k, v in res.items()},
           "exposed_ms": {"sequential": round(exposed_seq, 3), "overlap": round(exposed_ovl, 3)},
           "hidden_fraction": round(1 - exposed_ovl / exposed_seq, 3) if exposed_seq > 0 else None,
           "overlap_ms_by_workgroup_cap": {str(c): round(v, 3) for c, v in capped.items()},
           "workgroup_cap": best_cap,
           "backward_gemm_tflop": round(gemm_flops / 1e12, 3),
           "runs_per_pass": len(reducer.launch_log()),
           "model": model})


def _overlap_model(torch, ddp, plan, p, table, backward, n_params, reps=5):
    """The overlapped step-time model (ddp_overlap_step_time) fed with this
    device's own timings: each parameter's ready time from a backward-only
    pass queued behind another (events after its gradients are written, from
    an event at the pass's start), each bucket's all-reduce
    time from its own launches. The model takes the all-reduces to run on a
    resource of their own; on one GPU they share compute units and HBM with
    the backward, which the measured exposed time includes. The same ready
    times with the latency-bandwidth ring time of each bucket on the page's
    example network (alpha 10 us, 50 GB/s) give what a real link would
    expose."""
    start = torch.cuda.Event(enable_timing=True)
    after = [torch.cuda.Event(enable_timing=True) for _ in range(n_params)]
    ready = [0.0] * n_params
    for _ in range(reps):
        # the timed pass queued behind an untimed one, as in back-to-back steps
        torch.cuda.synchronize()
        backward(False)
        backward(False, (start, after))
        torch.cuda.synchronize()
        for i, e in enumerate(after):
            ready[i] += start.elapsed_time(e) * 1e-3 / reps
    nb = plan.num_buckets
    timer = ddp.CallTimer(pairs=nb * reps)
    ids = [[] for _ in range(nb)]
    for _ in range(reps):
        for b in range(nb):
            ids[b].append(timer.arm())
            ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
    torch.cuda.synchronize()
    btime = [sum(timer.elapsed_ms(k) for k in ids[b]) * 1e-3 / reps for b in range(nb)]
    step, exposed = ddp.overlap_step_time(plan, ready, btime)
    alpha, beta = 10e-6, 1 / 50e9
    nbytes = [plan.bucket_numel(b) * plan.elem_bytes for b in range(nb)]
    net = [ddp.schedule_time("ring", p, m, alpha, beta) for m in nbytes]
    nstep, nexp = ddp.overlap_step_time(plan, ready, net)
    return {"inputs": "ready times: backward-only pass on the device; bucket times: "
                      "per-bucket all-reduce launches on the device",
            "backward_ms": round(max(ready) * 1e3, 3),
            "allreduce_ms_sum": round(sum(btime) * 1e3, 3),
            "step_ms": round(step * 1e3, 3), "exposed_ms": round(exposed * 1e3, 3),
            "network_alpha10us_50GBps": {"allreduce_ms_sum": round(sum(net) * 1e3, 3),
                                         "step_ms": round(nstep * 1e3, 3),
                                         "exposed_ms": round(nexp * 1e3, 3)}}


def bench_crossover(torch, ddp, W, dev, args):
    """Ring versus the logarithmic schedules on 4 ranks, step by step (one
    launch per step: the launch is the simulated message round, so its
    latency plays alpha and device-memory time plays beta), from 1 KB to
    64 MB per rank. Fits alpha and beta to the ring's times, predicts the
    ring / recursive-doubling crossover with the latency-bandwidth model,
    and reports where the measured times cross."""
    import numpy as np

    p = 4
    sizes = [1 << k for k in range(8, 25)]  # fp32 elements: 1 KB .. 64 MB per rank
    scheds = ["ring", "recursive_doubling", "rabenseifner", "tree"]
    nmax = sizes[-1]
    arena = [W.normal_torch(nmax, 1.0, 44, r, dev) for r in range(p)]
    table = {}
    for n in sizes:
        bufs = [a[:n] for a in arena]
        reps = 200 if n * 4 <= (1 << 20) else (40 if n * 4 <= (1 << 24) else 10)
        row = {}
        for sch in scheds:
            for steps in (True, False):
                fn = (lambda b=bufs, s=sch, st=steps:
                      ddp.allreduce_sim(b, s, st, avg="world"))
                for _ in range(3):
                    fn()
                _, dms = _timed_calls(torch, ddp, [fn], reps, wall=False)
                row[f"{sch}{'_steps' if steps else '_fused'}_us"] = round(dms * 1e3, 2)
        table[n * 4] = row
        log(f"crossover: {n * 4} bytes done")
    # alpha, beta from the ring's step form: t = 2(p-1)(alpha + beta M / p)
    xs = np.array([float(m) for m in table])
    ts = np.array([table[m]["ring_steps_us"] * 1e-6 for m in table])
    A = np.stack([np.full_like(xs, 2.0 * (p - 1)), 2.0 * (p - 1) * xs / p], axis=1)
    (alpha, beta), *_ = np.linalg.lstsq(A, ts, rcond=None)
    lg = np.log2(p)
    mstar = (alpha / beta) * (2 * (p - 1) - lg) / (lg - 2 * (p - 1) / p)
    cross = None
    ms = sorted(table)
    for a, b in zip(ms, ms[1:]):
        da = table[a]["recursive_doubling_steps_us"] - table[a]["ring_steps_us"]
        db = table[b]["recursive_doubling_steps_us"] - table[b]["ring_steps_us"]
        if da < 0 <= db:
            # log-linear interpolation of where the difference changes sign
            f = -da / (db - da)
            cross = float(np.exp(np.log(a) + f * (np.log(b) - np.log(a))))
            break
    pick = {m: min(scheds, key=lambda s: table[m][f"{s}_steps_us"]) for m in ms}
    graph = _crossover_graphs(torch, ddp, arena, sizes, p, np)
    _line("ring vs recursive-doubling crossover, p=4, step-by-step schedules",
          cross if cross is not None else float("nan"), "bytes per rank",
          "crossover sweep: p=4, one fp32 tensor of 1 KB .. 64 MB per rank, average by p, "
          "each schedule step by step (one launch per message round) and fused",
          {"higher_is_better": False,
           "model": {"alpha_us": round(alpha * 1e6, 3), "beta_ns_per_byte": round(beta * 1e9, 6),
                     "predicted_crossover_bytes": round(float(mstar), 1)},
           "fastest_step_schedule": {str(m): pick[m] for m in ms},
           "the_three_sizes": {str(m): table[m] for m in (1 << 10, 1 << 20, 1 << 24)},
           "sweep_us": {str(m): table[m] for m in ms},
           "graph_replay": graph})


def _crossover_graphs(torch, ddp, arena, sizes, p, np):
    """The ring and recursive doubling step by step, each call captured once
    in a HIP graph and replayed: the per-step cost without the host's launch
    path. Fits alpha and beta to the replayed ring as above and finds where
    the replayed schedules cross."""
    times = {}
    side = torch.cuda.Stream()
    for n in sizes:
        bufs = [a[:n] for a in arena]
        reps = 200 if n * 4 <= (1 << 20) else (40 if n * 4 <= (1 << 24) else 10)
        for sch in ("ring", "recursive_doubling"):
            fn = lambda b=bufs, s=sch: ddp.allreduce_sim(b, s, True, avg="world")  # noqa: E731
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            g.replay()
            torch.cuda.synchronize()
            times[(n * 4, sch)] = _events_ms(torch, g.replay, reps) * 1e3
            del g
    ms = sorted({m for m, _ in times})
    xs = np.array([float(m) for m in ms])
    ts = np.array([times[(m, "ring")] * 1e-6 for m in ms])
    A = np.stack([np.full_like(xs, 2.0 * (p - 1)), 2.0 * (p - 1) * xs / p], axis=1)
    (alpha, beta), *_ = np.linalg.lstsq(A, ts, rcond=None)
    lg = np.log2(p)
    mstar = (alpha / beta) * (2 * (p - 1) - lg) / (lg - 2 * (p - 1) / p)
    cross = None
    for a, b in zip(ms, ms[1:]):
        da = times[(a, "recursive_doubling")] - times[(a, "ring")]
        db = times[(b, "recursive_doubling")] - times[(b, "ring")]
        if da < 0 <= db:
            f = -da / (db - da)
            cross = float(np.exp(np.log(a) + f * (np.log(b) - np.log(a))))
            break
    return {"crossover_bytes": cross,
            "model": {"alpha_us": round(alpha * 1e6, 3),
                      "beta_ns_per_byte": round(beta * 1e9, 6),
                      "predicted_crossover_bytes": round(float(mstar), 1)},
            "us": {str(m): {"ring_steps_us": round(times[(m, "ring")], 2),
                            "recursive_doubling_steps_us":
                                round(times[(m, "recursive_doubling")], 2)} for m in ms}}


def bench_sync(torch, ddp, W, dev, args):
    """The init-time synchronisation of the GPT-2-small parameters (148 fp32
    tensors, 124,439,808 elements per rank) from rank 0 to 8 ranks, coalesced
    into 250 MiB buckets, plus a per-forward buffer broadcast of BatchNorm-like
    statistics (two fp32 buffers per layer and an int64 counter)."""
    p = 8
    sizes = [W.numel(s) for _, s in W.gpt2_small_params()]
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 63) // 64 * 64
    arenas = [W.normal_torch(off, 1e-3, 2, r, dev) for r in range(p)]
    views = [[a[o:o + n] for o, n in zip(offs, sizes)] for a in arenas]
    plan = ddp.ddp_coalesce_plan(sizes, 4, ddp.BROADCAST_BUCKET_BYTES).upload(dev)
    table = ddp.grad_pointer_table(views, dev)
    fn = lambda: ddp.ddp_broadcast_coalesced(plan, table, p, 0)  # noqa: E731
    for _ in range(args.warmup):
        fn()
    wall, dms = _timed_calls(torch, ddp, [fn], args.steps)
    S = sum(sizes) * 4
    hbm = p * S
    st = fn()
    # the same ranks' whole arenas through broadcast_sim (one flat buffer per
    # rank, the fan-out copy): the same access pattern without the plan
    flat = [lambda: ddp.broadcast_sim(arenas, src=0)]
    flat[0]()
    _, fdms = _timed_calls(torch, ddp, flat, args.steps, wall=False)
    fbytes = p * arenas[0].numel() * 4
    # per-forward buffer broadcast: 12 layers x (running mean, running var)
    # of 3072 fp32 each, plus an int64 counter per layer
    bn = [[torch.randn(3072, device=dev) for _ in range(24)] +
          [torch.zeros(1, dtype=torch.int64, device=dev) for _ in range(12)] for _ in range(p)]
    groups = {}
    for i, t in enumerate(bn[0]):
        groups.setdefault(t.element_size(), []).append(i)
    calls = []
    keep = []
    for eb, idx in sorted(groups.items()):
        bplan = ddp.ddp_coalesce_plan([bn[0][i].numel() for i in idx], eb).upload(dev)
        btab = ddp.grad_pointer_table([[bn[r][i] for i in idx] for r in range(p)], dev)
        keep.append((bplan, btab))
        calls.append(lambda bp=bplan, bt=btab: ddp.ddp_broadcast_coalesced(bp, bt, p, 0))
    for c in calls:
        c()
    bwall, bdms = _timed_calls(torch, ddp, calls, max(args.steps, 50))
    _line("parameter sync GB/s per rank, p=8, GPT-2-small fp32 parameters from rank 0",
          S / (wall * 1e-3) / 1e9, "GB/s",
          "init-time sync: 148 fp32 GPT-2-small parameter tensors (124,439,808 elements per "
          "rank) broadcast from rank 0 to 8 ranks in 250 MiB coalesced buckets",
          {"ms": round(wall, 3), "kernel_ms": round(dms, 3), "buckets": plan.num_buckets,
           "launches": plan.num_buckets,
           "kernel_hbm_GBps": round(hbm / (dms * 1e-3) / 1e9, 1),
           "kernel_frac_of_8TBps": round(hbm / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "tree_messages": st.messages, "tree_rounds": st.steps,
           "broadcast_sim_of_the_arenas": {
               "kernel_ms": round(fdms, 3),
               "kernel_hbm_GBps": round(fbytes / (fdms * 1e-3) / 1e9, 1),
               "kernel_frac_of_8TBps": round(fbytes / (fdms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
           "buffer_broadcast": {"tensors": 36, "groups": len(calls),
                                "us_per_forward": round(bwall * 1e3, 2),
                                "kernel_us_per_forward": round(bdms * 1e3, 2)}})


def bench_ceilings(torch, ddp, W, dev, args):
    """Device-memory ceilings by access pattern, measured with the library's
    own kernels (and torch's fill for a single write stream): how much a
    kernel's speed depends on how many buffers each wave reads and writes at
    the same offset. A copy is broadcast_sim between 2 ranks; 1 read to p-1
    writes is broadcast_sim at p; p reads to 1 write is reduce_scatter_sim;
    2 reads to 1 write and 1 to 1 are the ring's steps; p to p is the fused
    all-reduce."""
    rows = {}

    def timed_ms(fn, reps):
        fn()
        _, dms = _timed_calls(torch, ddp, [fn], reps, wall=False)
        return dms

    for p, mib in ((2, 1024), (8, 1024), (64, 128)):
        n = mib * (1 << 20) // 4
        bufs = [torch.full((n,), float(r), device=dev) for r in range(p)]
        S = n * 4
        ms = timed_ms(lambda: ddp.broadcast_sim(bufs, src=0), args.steps)
        rows[f"broadcast_sim p={p}, {mib} MiB per rank: 1 read, {p - 1} writes"] = p * S / ms / 1e6
        outs = [torch.empty(n // p, device=dev) for _ in range(p)]
        ms = timed_ms(lambda: ddp.reduce_scatter_sim(bufs, outs), args.steps)
        rows[f"reduce_scatter_sim p={p}: {p} reads, 1 write"] = (p + 1) * S / ms / 1e6
        ms = timed_ms(lambda: ddp.ring_allreduce_sim(bufs, avg="world"), args.steps)
        rows[f"ring_allreduce_sim fused p={p}: {p} reads, {p} writes"] = 2 * p * S / ms / 1e6
        if p == 8:
            rs = [lambda: ddp.ring_allreduce_sim_steps(bufs, 0, 1, avg="world")]
            ms = timed_ms(rs[0], args.steps)
            rows["ring reduce-scatter step p=8: 2 reads, 1 write"] = 3 * S / ms / 1e6
            ag = [lambda: ddp.ring_allreduce_sim_steps(bufs, p - 1, 1, avg="world")]
            ms = timed_ms(ag[0], args.steps)
            rows["ring all-gather step p=8: 1 read, 1 write"] = 2 * S / ms / 1e6
        del bufs, outs
        torch.cuda.empty_cache()
    a = torch.empty(1 << 28, device=dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    a.fill_(1.0)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        a.fill_(2.0)
    e1.record()
    torch.cuda.synchronize()
    rows["torch fill_ of 1 GiB: 1 write"] = (1 << 30) / (e0.elapsed_time(e1) / args.steps) / 1e6
    del a
    _line("device-memory GB/s by access pattern (library kernels)",
          rows["broadcast_sim p=2, 1024 MiB per rank: 1 read, 1 writes"], "GB/s",
          "ceilings: the library's copy, fan-out, fan-in, ring-step and fused kernels on 2, 8 "
          "and 64 ranks of 1 GiB / 1 GiB / 128 MiB, and a single-stream fill",
          {"GBps": {k: round(v, 1) for k, v in rows.items()},
           "frac_of_8TBps": {k: round(v / HBM_PEAK_GBPS, 4) for k, v in rows.items()}})


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
    other = {"ragged-ring-p4": bench_ragged, "llama7b-bf16-p8": bench_llama,
             "latency-p64": bench_latency, "cost-model-p64": bench_costmodel,
             "collectives-p8": bench_collectives_p8,
             "overlap-gpt2-p8": bench_overlap, "crossover-p4": bench_crossover,
             "sync-gpt2-p8": bench_sync, "ceilings": bench_ceilings}
    if args.workload in other:
        log(f"workload {args.workload}")
        other[args.workload](torch, ddp, W, dev, args)
        return
    log("building workload")
    wl = Workload(torch, ddp, W, dev)
    p, S = wl.p, wl.S
    if not args.no_cpu_baseline:
        # the oracle's inputs: the values the GPU starts from
        wl.host_arenas = [host_copy(a) for a in wl.arenas]
    ws = {}
    modes = [args.mode] + ([] if args.no_compare else
                           [m for m in ("batched", "inplace", "copy") if m != args.mode])
    if "copy" in modes:
        wl.ensure_bucket_buffers(torch, dev)
        if args.algo == "ring":
            for b, n in enumerate(wl.nb):
                need = ddp.ring_allreduce_sim_workspace(p, n, 0, "ring")
                ws[b] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    torch.cuda.synchronize()

    results = {}
    for mode in modes:
        log(f"{mode}: warmup {args.warmup}, timing {args.steps} steps")
        ms, kernels, ms_ev = timed(torch, ddp, wl, mode, args.algo, args.steps, args.warmup, ws)
        results[mode] = (ms, kernels, ms_ev)
        log(f"{mode}: {ms:.3f} ms/step ({ms_ev:.3f} with kernel events); " + "; ".join(
            f"{k} {v['avg_us']} us avg, {v['GBps']} GB/s" for k, v in kernels.items()))

    ms, kernels, ms_ev = results[args.mode]
    dominant = max(kernels.items(), key=lambda kv: kv[1]["ms"])
    dname, d = dominant
    bus = S * 2 * (p - 1) / p / (ms * 1e-3) / 1e9
    step_bytes = 6 * p * S if args.mode == "copy" else 2 * p * S
    result = {
        "metric": METRIC,
        "value": round(bus, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_with_kernel_events": round(ms_ev, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("gpt2-small gradients: 148 fp32 tensors, 124,439,808 elements per "
                         "rank, p=8 simulated ranks, 25 MiB buckets + 1 MiB first bucket "
                         "(13 buckets), average by p; step = flatten + ring all-reduce + "
                         "unflatten of every bucket"),
            "step_kernels": {
                "batched": "one ddp_allreduce_buckets launch for the run of all 13 ready "
                           "buckets (each with its own ring chunks)",
                "inplace": "one ddp_allreduce_bucket launch per bucket",
                "copy": f"ddp_flatten + ring_allreduce_sim({args.algo}) + ddp_unflatten "
                        "per bucket"}[args.mode],
            "p": p, "buckets": wl.plan.num_buckets, "bytes_per_rank": S,
            # where each rank's arena starts, modulo 2 MiB (the layout the
            # kernel's speed was compared across)
            "arena_base_mod_2MiB": [a.data_ptr() % (2 << 20) for a in wl.arenas],
        },
        "hbm_frac_step": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels": kernels,
        "roofline": {
            "kernel": dname,
            "bound": "hbm",
            "achieved": d["GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(d["GBps"] / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(dname),
            "avg_launch_us": d["avg_us"],
            "bytes_per_launch": d["bytes"] // d["launches"],
        },
    }
    for mode, (mms, mk, mev) in results.items():
        if mode != args.mode:
            sb = 6 * p * S if mode == "copy" else 2 * p * S
            result[f"{mode}_step"] = {
                "ms_per_step": round(mms, 4),
                "ms_per_step_with_kernel_events": round(mev, 4),
                "bus_GBps": round(S * 2 * (p - 1) / p / (mms * 1e-3) / 1e9, 2),
                "hbm_frac_step": round(sb / (mms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "kernels": mk,
            }
    # the practical roofline: the library's own copy (a broadcast between two
    # ranks of 1 GiB reads one buffer and writes the other once)
    cp = [torch.ones(1 << 28, device=dev), torch.empty(1 << 28, device=dev)]
    ccall = [lambda: ddp.broadcast_sim(cp, src=0)]
    ccall[0]()
    _, cdms = _timed_calls(torch, ddp, ccall, 10, wall=False)
    copy_gbps = 2 * (1 << 30) / (cdms * 1e-3) / 1e9
    result["practical_ceiling"] = {
        "copy_GBps": round(copy_gbps, 1),
        "kernel": "fanout_copy_kernel (broadcast_sim between 2 ranks of 1 GiB: 1 read, 1 write)",
        "headline_frac_of_copy": round(d["GBps"] / copy_gbps, 4)}
    del cp
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 1024 * 1024 // 4
        a = torch.ones(n, device=dev)
        b2 = torch.empty(n, device=dev)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            b2.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / reps
        result["copy_calibration"] = {"bytes": 2 * n * 4, "ms": round(cms, 4),
                                      "GBps": round(2 * n * 4 / (cms * 1e-3) / 1e9, 1)}
        del a, b2
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(W, wl, args.cpu_buckets)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
