"""Latency-bandwidth (Hockney alpha-beta) cost model of the collectives.

TEST INFRASTRUCTURE / reporting only; part of the oracle package.

The page "Data parallelism" (zerotofrontier), sections "Ring all-reduce,
derived", "Latency, trees, and choosing an algorithm" and "When data
parallelism stops scaling", derives these times, but its display equations
were lost when the page was extracted to text. They are reconstructed here
from the surrounding prose and pinned to the numbers the page prints (see
tests/golden/cost_model.json):

  naive (root) all-reduce  2 (p-1) M / B          the root receives and sends (p-1)M
  ring all-reduce          2 (p-1) (alpha + beta M / p)
  recursive doubling       log2(p) (alpha + beta M)
  crossover M*             t_ring == t_rd solved for M
  overlap condition        backward 4 N n_tok / F  >=  all-reduce 4 N / B
                           so n_tok >= F / B

Bytes per rank: all-reduce 2 (p-1) M / p; reduce-scatter or all-gather alone
(p-1) M / p ("Ring all-reduce, derived"; "Collective Ops From Scratch").
"""
from __future__ import annotations

import math


def collective_bytes(op: str, M: float, p: int) -> float:
    """Bytes each rank sends for one collective on an M-byte buffer."""
    if op == "allreduce":
        return 2.0 * (p - 1) * M / p
    if op in ("reduce_scatter", "allgather"):
        return (p - 1) * M / p
    if op == "naive_allreduce_root":
        return (p - 1) * M
    raise ValueError(op)


def naive_allreduce_time(M: float, p: int, bandwidth: float) -> float:
    """Root gathers (p-1)M bytes and sends (p-1)M bytes back."""
    return 2.0 * (p - 1) * M / bandwidth


def allreduce_time(M: float, p: int, alpha: float, beta: float, algo: str) -> float:
    """Hockney-model time of one all-reduce of M bytes over p ranks."""
    if algo == "ring":
        return 2.0 * (p - 1) * (alpha + beta * M / p)
    if algo == "rd":
        return math.log2(p) * (alpha + beta * M)
    raise ValueError(algo)


def ring_crossover(p: int, alpha: float, beta: float) -> float:
    """Message size above which the ring beats recursive doubling."""
    lg = math.log2(p)
    return (alpha / beta) * (2.0 * (p - 1) - lg) / (lg - 2.0 * (p - 1) / p)


def overlap_tokens(flops_per_s: float, bandwidth: float) -> float:
    """Tokens per GPU per step needed to hide the all-reduce under backward."""
    return flops_per_s / bandwidth


def ddp_step_time(grads, bucket_cap, p, alpha, beta):
    """Step time with bucketed, overlapped all-reduce ("Data parallelism",
    section "Overlapping communication with the backward pass").

    grads: [(bytes, t_ready)] in the order backward produces them. Buckets
    are filled in that order and closed once they reach bucket_cap bytes.
    A bucket's ring all-reduce starts when its last gradient is ready and
    the previous bucket's all-reduce has finished, and takes
    2(p-1)(alpha + beta * M_b / p). Returns (step time, exposed time), the
    exposed time being what sticks out past the end of backward.
    """
    end_bwd = max((t for _, t in grads), default=0.0)
    buckets = []
    size, ready = 0.0, 0.0
    for n, t in grads:
        if size >= bucket_cap and size > 0:
            buckets.append((size, ready))
            size, ready = 0.0, 0.0
        size += n
        ready = max(ready, t)
    if size > 0 or not buckets:
        buckets.append((size, ready))
    finish = 0.0
    for m, t in buckets:
        start = max(t, finish)
        finish = start + allreduce_time(m, p, alpha, beta, "ring")
    step = max(end_bwd, finish)
    return step, step - end_bwd
