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

schedule_time prices the literal schedules of the oracle's orc_allreduce
message by message (one alpha per step, the largest message of a step for
the beta term). For p a power of two it is the page's formula for each
schedule: ring 2(p-1)(alpha + beta M/p); recursive doubling
log2 p (alpha + beta M); recursive halving/doubling 2 log2 p alpha +
2 (p-1)/p M beta. For other p, two whole-buffer steps (an extra rank's data
in, the result back out) are added to the power-of-two core, the reading
the oracle takes. The tree all-reduce (reduce up, broadcast down the
doubling tree) takes 2 ceil(log2 p) whole-buffer steps.
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


SCHEDULES = ("ring", "recursive_doubling", "rabenseifner", "tree")


def _pow2_floor(p: int) -> int:
    q = 1
    while q * 2 <= p:
        q *= 2
    return q


def schedule_time(schedule: str, M: float, p: int, alpha: float, beta: float) -> float:
    """Hockney-model time of one all-reduce of M bytes under a schedule."""
    if p == 1:
        return 0.0
    q = _pow2_floor(p)
    k = int(math.log2(q))
    extra = 2 * (alpha + beta * M) if q < p else 0.0
    if schedule == "ring":
        return allreduce_time(M, p, alpha, beta, "ring")
    if schedule == "recursive_doubling":
        return k * (alpha + beta * M) + extra
    if schedule == "rabenseifner":
        return 2 * k * alpha + 2.0 * (q - 1) / q * M * beta + extra
    if schedule == "tree":
        K = math.ceil(math.log2(p))
        return 2 * K * (alpha + beta * M)
    raise ValueError(schedule)


def choose_schedule(p: int, M: float, alpha: float, beta: float,
                    candidates=("ring", "recursive_doubling")) -> str:
    """The candidate with the smallest modelled time; ties go to the one
    listed first ("Latency, trees, and choosing an algorithm": libraries pick
    per call from the message size)."""
    best, best_t = None, None
    for c in candidates:
        t = schedule_time(c, M, p, alpha, beta)
        if best is None or t < best_t:
            best, best_t = c, t
    return best
