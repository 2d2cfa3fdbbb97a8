"""CPU oracle for the bucketed data-parallel gradient-synchronisation path.

TEST INFRASTRUCTURE ONLY. The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only code allowed to import this
package. The product library (``bucketed_gradient_all_ddp_amd``) never
imports, loads or calls it, and the two share no code: the only thing both
sides use is the seeded input generator in
``bucketed_gradient_all_ddp_amd.workloads``, which holds none of the method's
arithmetic.

The arithmetic lives in ``ring_oracle.c`` (plain C, one thread, IEEE fp32,
no FMA contraction, no flush-to-zero), built here with gcc and called through
ctypes. This module only marshals numpy arrays, plus the integer geometry of
chunks for the sampled-element checks.

Pages cited (by title and section):
  "PyTorch DDP Deep Dive" -- bucket assignment, the reducer's copy into the
      bucket, the copy back in finalize_backward.
  "Collective Ops From Scratch" -- ring allreduce in two passes, padding,
      reduce_scatter pre-rotation, allgather rotations, doubling-tree
      broadcast, the 1e-5 gloo check.
  "Data parallelism" (zerotofrontier) -- ring all-reduce derived, chunk
      ownership (q+1) mod p, bytes per rank, averaging by tokens; recursive
      doubling and recursive halving/doubling ("Latency, trees, and choosing
      an algorithm").

Parity pins for every function are in tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ring_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = [
    "-O2", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math",
    "-ffp-contract=off", "-fPIC", "-shared",
]

AVG_MODES = {"none": 0, "world": 1, "tokens": 2}
DTYPES = {"f32": 0, "bf16": 1}

PHASE_REDUCE_SCATTER = 0
PHASE_ALLGATHER = 1
PHASE_BROADCAST = 2
PHASE_EXCHANGE = 3
PHASE_FOLD_IN = 4
PHASE_FOLD_OUT = 5
PHASE_REDUCE = 6

SCHEDULES = {"ring": 0, "recursive_doubling": 1, "rabenseifner": 2, "tree": 3}

_lib = None


def build() -> str:
    """Compile ring_oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


@dataclass(frozen=True)
class Message:
    phase: int
    step: int
    src: int
    dst: int
    chunk: int
    bytes: int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.orc_bucket_plan.argtypes = [P, i32, i32, i64, i64, P, P, P, P, P]
    lib.orc_bucket_plan.restype = ctypes.c_int
    lib.orc_bucket_plan_ordered.argtypes = [P, i32, P, i32, i64, i64, P, P, P, P, P]
    lib.orc_bucket_plan_ordered.restype = ctypes.c_int
    lib.orc_coalesce_plan.argtypes = [P, i32, i32, i64, P, P, P, P, P]
    lib.orc_coalesce_plan.restype = ctypes.c_int
    lib.orc_broadcast_coalesced.argtypes = [P, P, i32, i32, i32, i64, i32, P, i64, P, P]
    lib.orc_broadcast_coalesced.restype = ctypes.c_int
    lib.orc_flatten.argtypes = [P, P, P, P, P, i32, i32, f32, P]
    lib.orc_flatten.restype = ctypes.c_int
    lib.orc_unflatten.argtypes = [P, P, P, P, P, i32, i32, P]
    lib.orc_unflatten.restype = ctypes.c_int
    lib.orc_ring_allreduce.argtypes = [P, i32, i64, i32, i32, P, i32, P, i64, P]
    lib.orc_ring_allreduce.restype = ctypes.c_int
    lib.orc_reduce_scatter.argtypes = [P, P, i32, i64, i32, i32, P, P, i64, P]
    lib.orc_reduce_scatter.restype = ctypes.c_int
    lib.orc_allgather.argtypes = [P, P, i32, i64, i32, P, i64, P]
    lib.orc_allgather.restype = ctypes.c_int
    lib.orc_broadcast.argtypes = [P, i32, i64, i32, i32, P, i64, P]
    lib.orc_broadcast.restype = ctypes.c_int
    lib.orc_fold_samples.argtypes = [P, P, i32, i64, i32, f32, P]
    lib.orc_fold_samples.restype = None
    lib.orc_f32_to_bf16_array.argtypes = [P, P, i64]
    lib.orc_f32_to_bf16_array.restype = None
    lib.orc_bf16_to_f32_array.argtypes = [P, P, i64]
    lib.orc_bf16_to_f32_array.restype = None
    lib.orc_avg_divisor.argtypes = [i32, i32, P, P]
    lib.orc_avg_divisor.restype = ctypes.c_int
    lib.orc_reducer_schedule.argtypes = [P, i32, i32, P, i32, P, P, P]
    lib.orc_reducer_schedule.restype = ctypes.c_int
    lib.orc_allreduce.argtypes = [P, i32, i64, i32, i32, P, i32, P, i64, P]
    lib.orc_allreduce.restype = ctypes.c_int
    lib.orc_tree_fold_samples.argtypes = [P, i32, i64, i32, i32, f32, P]
    lib.orc_tree_fold_samples.restype = i32
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc == -2:
        raise ValueError(f"{what}: element count not divisible by world size")
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_table(arrays: Sequence[Optional[np.ndarray]]) -> np.ndarray:
    """Addresses of the arrays (0 for None: parameters a call does not touch)."""
    return np.array([0 if a is None else a.ctypes.data for a in arrays], dtype=np.uintp)


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return 0
    if arr.dtype == np.uint16:
        return 1
    raise TypeError("oracle buffers are float32 or uint16 (bf16 bit patterns)")


def _tokens_array(tokens, p: int) -> Optional[np.ndarray]:
    if tokens is None:
        return None
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    if t.shape != (p,):
        raise ValueError("tokens must hold one count per rank")
    return t


def _messages(buf: np.ndarray, count: int) -> List[Message]:
    return [
        Message(int(m["phase"]), int(m["step"]), int(m["src"]), int(m["dst"]),
                int(m["chunk"]), int(m["bytes"]))
        for m in buf[:count]
    ]


_MSG_DTYPE = np.dtype([
    ("phase", np.int32), ("step", np.int32), ("src", np.int32),
    ("dst", np.int32), ("chunk", np.int32), ("reserved", np.int32),
    ("bytes", np.int64),
])


# ---------------------------------------------------------------------------
# bf16 conversion
# ---------------------------------------------------------------------------

def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 (returned as uint16 bit patterns)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_f32_to_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    lib = _load()
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib.orc_bf16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def avg_divisor(avg: str, p: int, tokens=None) -> float:
    """The fp32 divisor used for averaging (1 when not averaging)."""
    lib = _load()
    t = _tokens_array(tokens, p)
    out = np.zeros(1, dtype=np.float32)
    rc = lib.orc_avg_divisor(AVG_MODES[avg], p, None if t is None else _ptr(t),
                             _ptr(out))
    _check(rc, "avg_divisor")
    return float(out[0])


# ---------------------------------------------------------------------------
# Bucket plan
# ---------------------------------------------------------------------------

@dataclass
class Plan:
    numel: np.ndarray          # int64[P], registration order
    elem_bytes: int
    fill_order: np.ndarray     # int32[P]
    bucket_begin: np.ndarray   # int32[B+1]
    offset: np.ndarray         # int64[P], element offset inside its bucket
    bucket_of: np.ndarray      # int32[P]

    @property
    def num_buckets(self) -> int:
        return len(self.bucket_begin) - 1

    def bucket_params(self, b: int) -> List[int]:
        lo, hi = self.bucket_begin[b], self.bucket_begin[b + 1]
        return [int(i) for i in self.fill_order[lo:hi]]

    def bucket_numel(self, b: int) -> int:
        return int(sum(int(self.numel[i]) for i in self.bucket_params(b)))

    def buckets(self) -> List[List[int]]:
        return [self.bucket_params(b) for b in range(self.num_buckets)]


def bucket_plan(numel: Sequence[int], elem_bytes: int = 4,
                bucket_cap_bytes: int = 25 * 1024 * 1024,
                first_bucket_cap_bytes: int = 1024 * 1024,
                order: Optional[Sequence[int]] = None) -> Plan:
    """Greedy bucketing with a small first bucket, walking the parameters in
    reverse registration order, or in `order` (a permutation: the order in
    which gradients became ready, for a rebuild)."""
    lib = _load()
    nm = np.ascontiguousarray(np.asarray(numel, dtype=np.int64))
    P = len(nm)
    fill = np.zeros(max(P, 1), dtype=np.int32)
    begin = np.zeros(P + 2, dtype=np.int32)
    offset = np.zeros(max(P, 1), dtype=np.int64)
    bucket_of = np.zeros(max(P, 1), dtype=np.int32)
    nb = np.zeros(1, dtype=np.int32)
    if order is None:
        rc = lib.orc_bucket_plan(_ptr(nm) if P else None, P, elem_bytes,
                                 bucket_cap_bytes, first_bucket_cap_bytes,
                                 _ptr(fill), _ptr(begin), _ptr(offset),
                                 _ptr(bucket_of), _ptr(nb))
    else:
        walk = np.ascontiguousarray(np.asarray(order, dtype=np.int32))
        if walk.shape != (P,):
            raise ValueError("order must list every parameter once")
        rc = lib.orc_bucket_plan_ordered(_ptr(nm) if P else None, P,
                                         _ptr(walk) if P else None, elem_bytes,
                                         bucket_cap_bytes, first_bucket_cap_bytes,
                                         _ptr(fill), _ptr(begin), _ptr(offset),
                                         _ptr(bucket_of), _ptr(nb))
    _check(rc, "bucket_plan")
    B = int(nb[0])
    return Plan(nm, elem_bytes, fill[:P].copy(), begin[:B + 1].copy(),
                offset[:P].copy(), bucket_of[:P].copy())


def coalesce_plan(numel: Sequence[int], elem_bytes: int,
                  cap_bytes: int = 250 * 1024 * 1024) -> Plan:
    """Buckets of a coalesced broadcast: list order, none past the cap unless
    one tensor alone is."""
    lib = _load()
    nm = np.ascontiguousarray(np.asarray(numel, dtype=np.int64))
    P = len(nm)
    fill = np.zeros(max(P, 1), dtype=np.int32)
    begin = np.zeros(P + 2, dtype=np.int32)
    offset = np.zeros(max(P, 1), dtype=np.int64)
    bucket_of = np.zeros(max(P, 1), dtype=np.int32)
    nb = np.zeros(1, dtype=np.int32)
    rc = lib.orc_coalesce_plan(_ptr(nm) if P else None, P, elem_bytes, cap_bytes,
                               _ptr(fill), _ptr(begin), _ptr(offset), _ptr(bucket_of),
                               _ptr(nb))
    _check(rc, "coalesce_plan")
    B = int(nb[0])
    return Plan(nm, elem_bytes, fill[:P].copy(), begin[:B + 1].copy(),
                offset[:P].copy(), bucket_of[:P].copy())


def broadcast_coalesced(tensors: Sequence[Sequence[np.ndarray]], root: int = 0,
                        cap_bytes: int = 250 * 1024 * 1024):
    """tensors[r][i] = rank r's copy of tensor i (one dtype). Returns
    (results in the same layout, message log, bucket of each tensor)."""
    lib = _load()
    p = len(tensors)
    n_t = len(tensors[0]) if p else 0
    work = [[np.array(t, copy=True).ravel() for t in row] for row in tensors]
    eb = work[0][0].itemsize if n_t else 4
    numel = np.array([work[0][i].size for i in range(n_t)], dtype=np.int64)
    for row in work:
        if [t.size for t in row] != list(numel):
            raise ValueError("every rank must hold the same tensor shapes")
    table = _ptr_table([t for row in work for t in row])
    cap = p * max(n_t, 1) + 1
    log = np.zeros(cap, dtype=_MSG_DTYPE)
    count = np.zeros(1, dtype=np.int64)
    bof = np.zeros(max(n_t, 1), dtype=np.int32)
    rc = lib.orc_broadcast_coalesced(_ptr(table), _ptr(numel) if n_t else None, n_t, p,
                                     eb, cap_bytes, root, _ptr(log), cap, _ptr(count),
                                     _ptr(bof))
    _check(rc, "broadcast_coalesced")
    return work, _messages(log, int(count[0])), [int(b) for b in bof[:n_t]]


def flatten(grads: Sequence[np.ndarray], plan: Plan, b: int,
            divisor: float = 1.0) -> np.ndarray:
    """One rank's flat bucket buffer for bucket b (grads indexed by param)."""
    lib = _load()
    dt = _dtype_code(grads[plan.bucket_params(b)[0]]) if plan.bucket_params(b) else 0
    arrs = [None if g is None else np.ascontiguousarray(g) for g in grads]
    for i in plan.bucket_params(b):
        if arrs[i].size != plan.numel[i]:
            raise ValueError(f"gradient {i} has the wrong size")
    table = _ptr_table(arrs)
    flat = np.zeros(plan.bucket_numel(b), dtype=np.float32 if dt == 0 else np.uint16)
    rc = lib.orc_flatten(_ptr(table), _ptr(plan.numel), _ptr(plan.fill_order),
                         _ptr(plan.bucket_begin), _ptr(plan.offset), b, dt,
                         divisor, _ptr(flat))
    _check(rc, "flatten")
    return flat


def unflatten(flat: np.ndarray, plan: Plan, b: int,
              grads: Sequence[np.ndarray]) -> None:
    """Copy bucket b's flat buffer back into the (writable) gradient arrays."""
    lib = _load()
    for i in plan.bucket_params(b):
        if grads[i] is None or not grads[i].flags.c_contiguous or grads[i].size != plan.numel[i]:
            raise ValueError(f"gradient {i} must be contiguous and sized")
    table = _ptr_table(grads)
    flat = np.ascontiguousarray(flat)
    rc = lib.orc_unflatten(_ptr(table), _ptr(plan.numel), _ptr(plan.fill_order),
                           _ptr(plan.bucket_begin), _ptr(plan.offset), b,
                           flat.itemsize, _ptr(flat))
    _check(rc, "unflatten")


# ---------------------------------------------------------------------------
# Collectives (literal simulations with a message log)
# ---------------------------------------------------------------------------

def ring_allreduce(bufs: Sequence[np.ndarray], avg: str = "none", tokens=None,
                   max_steps: int = -1, want_log: bool = True
                   ) -> Tuple[List[np.ndarray], List[Message]]:
    """Ring all-reduce of p rank arrays; returns (results, message log).

    Inputs are not modified. max_steps >= 0 stops after that many of the
    2(p-1) ring steps and returns the partial state (trimmed to n).
    """
    lib = _load()
    p = len(bufs)
    work = [np.array(b, copy=True).ravel() for b in bufs]
    n = work[0].size if p else 0
    dt = _dtype_code(work[0])
    for w in work:
        if w.size != n or w.dtype != work[0].dtype:
            raise ValueError("rank buffers must match in size and dtype")
    t = _tokens_array(tokens, p)
    cap = 2 * p * max(p - 1, 0) if want_log else 0
    log = np.zeros(max(cap, 1), dtype=_MSG_DTYPE)
    count = np.zeros(1, dtype=np.int64)
    table = _ptr_table(work)
    rc = lib.orc_ring_allreduce(_ptr(table), p, n, dt, AVG_MODES[avg],
                                None if t is None else _ptr(t), max_steps,
                                _ptr(log) if want_log else None, cap,
                                _ptr(count))
    _check(rc, "ring_allreduce")
    return work, (_messages(log, int(count[0])) if want_log else [])


def reduce_scatter(bufs: Sequence[np.ndarray], avg: str = "none", tokens=None
                   ) -> Tuple[List[np.ndarray], List[Message]]:
    """Pre-rotated ring reduce-scatter: rank r returns the sum of chunk r."""
    lib = _load()
    p = len(bufs)
    ins = [np.ascontiguousarray(b).ravel() for b in bufs]
    n = ins[0].size
    dt = _dtype_code(ins[0])
    if n % p != 0:
        raise ValueError("reduce_scatter: element count not divisible by world size")
    C = n // p
    outs = [np.zeros(C, dtype=ins[0].dtype) for _ in range(p)]
    t = _tokens_array(tokens, p)
    cap = p * max(p - 1, 0)
    log = np.zeros(max(cap, 1), dtype=_MSG_DTYPE)
    count = np.zeros(1, dtype=np.int64)
    tin, tout = _ptr_table(ins), _ptr_table(outs)
    rc = lib.orc_reduce_scatter(_ptr(tin), _ptr(tout),
                                p, n, dt, AVG_MODES[avg],
                                None if t is None else _ptr(t), _ptr(log), cap,
                                _ptr(count))
    _check(rc, "reduce_scatter")
    return outs, _messages(log, int(count[0]))


def allgather(shards: Sequence[np.ndarray]
              ) -> Tuple[List[np.ndarray], List[Message]]:
    """Ring all-gather: every rank gets the rank-ordered concatenation."""
    lib = _load()
    p = len(shards)
    ins = [np.ascontiguousarray(s).ravel() for s in shards]
    C = ins[0].size
    outs = [np.zeros(p * C, dtype=ins[0].dtype) for _ in range(p)]
    cap = p * max(p - 1, 0)
    log = np.zeros(max(cap, 1), dtype=_MSG_DTYPE)
    count = np.zeros(1, dtype=np.int64)
    tin, tout = _ptr_table(ins), _ptr_table(outs)
    rc = lib.orc_allgather(_ptr(tin), _ptr(tout), p, C,
                           ins[0].itemsize, _ptr(log), cap, _ptr(count))
    _check(rc, "allgather")
    return outs, _messages(log, int(count[0]))


def broadcast(bufs: Sequence[np.ndarray], src: int = 0
              ) -> Tuple[List[np.ndarray], List[Message]]:
    """Doubling-tree broadcast of bufs[src] to every rank."""
    lib = _load()
    p = len(bufs)
    work = [np.array(b, copy=True).ravel() for b in bufs]
    n = work[0].size
    cap = max(p - 1, 0)
    log = np.zeros(max(cap, 1), dtype=_MSG_DTYPE)
    count = np.zeros(1, dtype=np.int64)
    table = _ptr_table(work)
    rc = lib.orc_broadcast(_ptr(table), p, n, work[0].itemsize, src,
                           _ptr(log), cap, _ptr(count))
    _check(rc, "broadcast")
    return work, _messages(log, int(count[0]))


def allreduce(bufs: Sequence[np.ndarray], schedule: str = "ring",
              avg: str = "none", tokens=None, want_log: bool = True
              ) -> Tuple[List[np.ndarray], List[Message]]:
    """All-reduce under a schedule ("ring", "recursive_doubling",
    "rabenseifner", "tree"); returns (results, message log). Inputs are not
    modified."""
    lib = _load()
    p = len(bufs)
    work = [np.array(b, copy=True).ravel() for b in bufs]
    n = work[0].size if p else 0
    dt = _dtype_code(work[0])
    for w in work:
        if w.size != n or w.dtype != work[0].dtype:
            raise ValueError("rank buffers must match in size and dtype")
    t = _tokens_array(tokens, p)
    cap = max(2 * p * max(p - 1, 0), 4 * p * 7, 1) if want_log else 0
    log = np.zeros(max(cap, 1), dtype=_MSG_DTYPE)
    count = np.zeros(1, dtype=np.int64)
    table = _ptr_table(work)
    rc = lib.orc_allreduce(_ptr(table), p, n, dt, AVG_MODES[avg],
                           None if t is None else _ptr(t), SCHEDULES[schedule],
                           _ptr(log) if want_log else None, cap, _ptr(count))
    _check(rc, "allreduce")
    return work, (_messages(log, int(count[0])) if want_log else [])


# ---------------------------------------------------------------------------
# The ring's result at sampled elements (for checks at full size)
# ---------------------------------------------------------------------------

def chunk_geometry(n: int, p: int) -> Tuple[int, int]:
    """(C, n_pad): equal chunks of ceil(n/p), zero padding at the end."""
    C = -(-n // p) if p else 0
    return C, C * p


def _fold(vals: np.ndarray, start: np.ndarray, p: int, divisor: float,
          do_divide: bool) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(vals, dtype=np.float32)
    s = np.ascontiguousarray(start, dtype=np.int64)
    k = s.size
    if v.shape != (k, p):
        raise ValueError("vals must be [samples, p]")
    out = np.empty(k, dtype=np.float32)
    lib.orc_fold_samples(_ptr(v), _ptr(s), p, k, 1 if do_divide else 0,
                         divisor, _ptr(out))
    return out


def allreduce_at(vals: np.ndarray, index: np.ndarray, n: int, avg: str = "none",
                 tokens=None) -> np.ndarray:
    """Ring all-reduce result at selected elements.

    vals[s, r] is rank r's input at element index[s] of an n-element buffer
    (float32, or uint16 bf16 patterns, which come back rounded to bf16).
    """
    vals = np.asarray(vals)
    p = vals.shape[1]
    C, _ = chunk_geometry(n, p)
    index = np.asarray(index, dtype=np.int64)
    if np.any(index < 0) or np.any(index >= n):
        raise ValueError("index out of range")
    start = index // C
    f = bf16_to_f32(vals) if vals.dtype == np.uint16 else vals
    out = _fold(f, start, p, avg_divisor(avg, p, tokens), avg != "none")
    return f32_to_bf16(out) if vals.dtype == np.uint16 else out


def reduce_scatter_at(vals: np.ndarray, index: np.ndarray, n: int,
                      avg: str = "none", tokens=None) -> np.ndarray:
    """Pre-rotated reduce-scatter result at selected input element indices.

    The result for input element i lands on rank i // C at position i % C.
    """
    vals = np.asarray(vals)
    p = vals.shape[1]
    if n % p != 0:
        raise ValueError("reduce_scatter: element count not divisible by world size")
    C = n // p
    index = np.asarray(index, dtype=np.int64)
    start = index // C + 1
    f = bf16_to_f32(vals) if vals.dtype == np.uint16 else vals
    out = _fold(f, start, p, avg_divisor(avg, p, tokens), avg != "none")
    return f32_to_bf16(out) if vals.dtype == np.uint16 else out


def tree_allreduce_at(vals: np.ndarray, schedule: str, avg: str = "none",
                      tokens=None) -> np.ndarray:
    """Result of a logarithmic schedule at selected elements: vals[s, r] is
    rank r's input at that element (float32, or uint16 bf16 patterns, which
    come back rounded to bf16). The value does not depend on the element's
    position."""
    lib = _load()
    vals = np.asarray(vals)
    p = vals.shape[1]
    f = np.ascontiguousarray(bf16_to_f32(vals) if vals.dtype == np.uint16 else vals,
                             dtype=np.float32)
    k = f.shape[0]
    out = np.empty(k, dtype=np.float32)
    _check(lib.orc_tree_fold_samples(_ptr(f), p, k, SCHEDULES[schedule],
                                     1 if avg != "none" else 0,
                                     avg_divisor(avg, p, tokens), _ptr(out)),
           "orc_tree_fold_samples")
    return f32_to_bf16(out) if vals.dtype == np.uint16 else out


# ---------------------------------------------------------------------------
# Reducer schedule
# ---------------------------------------------------------------------------

def reducer_schedule(plan: Plan, order: Sequence[int]):
    """Buckets launched by each ready mark, as (mark index, first bucket,
    count) for every mark that launches something, and the total launched
    (the number of buckets when every bucket became ready)."""
    lib = _load()
    o = np.ascontiguousarray(np.asarray(order, dtype=np.int32))
    m = o.size
    first = np.zeros(max(m, 1), dtype=np.int32)
    count = np.zeros(max(m, 1), dtype=np.int32)
    total = np.zeros(1, dtype=np.int32)
    bucket_of = np.ascontiguousarray(plan.bucket_of, dtype=np.int32)
    rc = lib.orc_reducer_schedule(_ptr(bucket_of) if bucket_of.size else None,
                                  bucket_of.size, plan.num_buckets,
                                  _ptr(o) if m else None, m, _ptr(first),
                                  _ptr(count), _ptr(total))
    _check(rc, "reducer_schedule")
    runs = [(k, int(first[k]), int(count[k])) for k in range(m) if count[k] > 0]
    return runs, int(total[0])
