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
