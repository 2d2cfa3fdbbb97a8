"""Python binding of libddpsim.so (include/ddpsim.h), argument marshalling only.

Each function takes torch tensors for device buffers, passes their
addresses, sizes and the current HIP stream to the C entry point of the same
name, and turns a non-zero status into DDPError. No arithmetic of the path
happens here: every step runs in the library's HIP kernels. PyTorch is used
only for device memory and streams.

The library is loaded on first use; if it has not been built, the call
raises ImportError rather than falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libddpsim.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
AVG = {"none": 0, "world": 1, "tokens": 2}
ALGO = {"fused": 0, "ring": 1}
MAX_RANKS = 64

STATUS = {
    0: "DDP_OK", 1: "DDP_EINVAL", 2: "DDP_ERANGE", 3: "DDP_EALIGN", 4: "DDP_EALIAS",
    5: "DDP_ENOTDIVISIBLE", 6: "DDP_ENOTREADY", 7: "DDP_EWORKSPACE", 8: "DDP_EHIP",
}

EXPORTS = [
    "ddp_strerror", "ddp_last_error", "ddp_version", "ddp_time_next_call",
    "ddp_bucket_plan", "ddp_plan_free", "ddp_plan_num_params", "ddp_plan_num_buckets",
    "ddp_plan_bucket_numel", "ddp_plan_bucket_size", "ddp_plan_bucket_params",
    "ddp_plan_param_bucket", "ddp_plan_param_offset", "ddp_plan_param_numel",
    "ddp_plan_elem_bytes", "ddp_plan_device_bytes",
    "ddp_plan_upload", "ddp_flatten", "ddp_unflatten",
    "ddp_plan_segment_bytes", "ddp_plan_upload_segments", "ddp_allreduce_bucket",
    "ddp_allreduce_buckets",
    "ddp_reducer_create", "ddp_reducer_free", "ddp_reducer_prepare", "ddp_reducer_mark_ready",
    "ddp_reducer_finalize", "ddp_reducer_launch_log", "ddp_reducer_ready_order",
    "ddp_reducer_set_max_workgroups", "ddp_bucket_plan_ordered", "ddp_coalesce_plan", "ddp_broadcast_coalesced",
    "ring_allreduce_sim", "ring_allreduce_sim_workspace", "ring_allreduce_sim_steps",
    "ring_allreduce_sim_noalloc",
    "allreduce_sim", "allreduce_sim_workspace", "ddp_schedule_time", "ddp_choose_schedule",
    "ddp_overlap_step_time",
    "reduce_scatter_sim", "allgather_sim", "broadcast_sim",
]

SCHEDULES = {"ring": 0, "recursive_doubling": 1, "rabenseifner": 2, "tree": 3}


class DDPError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{func}: {self.name}: {detail}")


class CommStats(ctypes.Structure):
    _fields_ = [
        ("steps", ctypes.c_int64),
        ("messages", ctypes.c_int64),
        ("bytes_sent_per_rank", ctypes.c_int64),
        ("bytes_recv_per_rank", ctypes.c_int64),
        ("total_bytes", ctypes.c_int64),
        ("hbm_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libddpsim.so and declare the C signatures (once)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime; loading it first makes this library
    # bind to that same runtime (one runtime per process, shared streams).
    import torch  # noqa: F401

    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    st = ctypes.c_int
    sig = {
        "ddp_strerror": ([st], ctypes.c_char_p),
        "ddp_last_error": ([], ctypes.c_char_p),
        "ddp_version": ([], ctypes.c_char_p),
        "ddp_time_next_call": ([vp, vp], st),
        "ddp_bucket_plan": ([vp, i32, i32, i64, i64, ctypes.POINTER(vp)], st),
        "ddp_plan_free": ([vp], None),
        "ddp_plan_num_params": ([vp], i32),
        "ddp_plan_num_buckets": ([vp], i32),
        "ddp_plan_bucket_numel": ([vp, i32], i64),
        "ddp_plan_bucket_size": ([vp, i32], i32),
        "ddp_plan_bucket_params": ([vp, i32, vp], st),
        "ddp_plan_param_bucket": ([vp, i32], i32),
        "ddp_plan_param_offset": ([vp, i32], i64),
        "ddp_plan_param_numel": ([vp, i32], i64),
        "ddp_plan_elem_bytes": ([vp], i32),
        "ddp_plan_device_bytes": ([vp], sz),
        "ddp_plan_upload": ([vp, vp, sz, vp], st),
        "ddp_flatten": ([vp, i32, i32, vp, vp, i32, f32, vp], st),
        "ddp_unflatten": ([vp, i32, i32, vp, vp, i32, vp], st),
        "ddp_plan_segment_bytes": ([vp, i32], sz),
        "ddp_plan_upload_segments": ([vp, i32, vp, sz, vp], st),
        "ddp_allreduce_bucket": ([vp, i32, i32, vp, i32, i32, vp, vp, vp], st),
        "ddp_allreduce_buckets": ([vp, i32, i32, i32, vp, i32, i32, vp, vp, vp], st),
        "ddp_reducer_create": ([vp, i32, vp, i32, i32, vp, vp, ctypes.POINTER(vp)], st),
        "ddp_reducer_free": ([vp], None),
        "ddp_reducer_prepare": ([vp], st),
        "ddp_reducer_mark_ready": ([vp, i32, vp], st),
        "ddp_reducer_finalize": ([vp, vp], st),
        "ddp_reducer_launch_log": ([vp, vp, vp, vp, i32], i32),
        "ddp_reducer_ready_order": ([vp, vp, i32], i32),
        "ddp_reducer_set_max_workgroups": ([vp, i32], st),
        "ddp_bucket_plan_ordered": ([vp, i32, vp, i32, i64, i64, ctypes.POINTER(vp)], st),
        "ddp_coalesce_plan": ([vp, i32, i32, i64, ctypes.POINTER(vp)], st),
        "ddp_broadcast_coalesced": ([vp, i32, vp, i32, vp, vp], st),
        "ring_allreduce_sim": ([vp, i32, i64, i32, i32, vp, i32, vp, sz, vp, vp], st),
        "ring_allreduce_sim_workspace": ([i32, i64, i32, i32], sz),
        "ring_allreduce_sim_noalloc": ([vp, i32, i64, i32, i32, vp, i32, vp, vp], st),
        "ring_allreduce_sim_steps": ([vp, i32, i64, i32, vp, i32, i32, vp], st),
        "allreduce_sim": ([vp, i32, i64, i32, i32, vp, i32, i32, vp, sz, vp, vp], st),
        "allreduce_sim_workspace": ([i32, i64, i32, i32, i32], sz),
        "ddp_schedule_time": ([i32, i32, ctypes.c_double, ctypes.c_double, ctypes.c_double],
                              ctypes.c_double),
        "ddp_choose_schedule": ([i32, i64, ctypes.c_double, ctypes.c_double, ctypes.c_uint32],
                                i32),
        "ddp_overlap_step_time": ([vp, vp, vp, vp, vp], st),
        "reduce_scatter_sim": ([vp, vp, i32, i64, i32, i32, vp, vp, vp], st),
        "allgather_sim": ([vp, vp, i32, i64, i32, vp, vp], st),
        "broadcast_sim": ([vp, i32, i64, i32, i32, vp, vp], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(status: int, func: str) -> None:
    if status != 0:
        detail = load_library().ddp_last_error().decode(errors="replace")
        raise DDPError(status, func, detail)


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _device_ptr(t) -> int:
    # the kernels dereference these addresses: host memory would fault the GPU
    if not t.is_cuda:
        raise TypeError("buffers must be device (cuda) tensors")
    return t.data_ptr()


def _ptrs(tensors: Sequence) -> ctypes.Array:
    return (ctypes.c_void_p * len(tensors))(*[_device_ptr(t) for t in tensors])


def _tokens(tokens, p: int):
    if tokens is None:
        return None
    if len(tokens) != p:
        raise ValueError("tokens needs one count per rank")
    return (ctypes.c_int64 * p)(*[int(t) for t in tokens])


def _numel_all(tensors: Sequence) -> int:
    n = tensors[0].numel()
    for t in tensors:
        if t.numel() != n or t.dtype != tensors[0].dtype or not t.is_contiguous():
            raise ValueError("rank buffers must be contiguous with equal size and dtype")
    return n


# ---------------------------------------------------------------------------
# Kernel timing (HIP events attached to one call's kernel dispatches)
# ---------------------------------------------------------------------------

class CallTimer:
    """A pool of HIP event pairs. arm() makes the next library call on this
    thread record its kernels' start and end on one pair; elapsed_ms() reads
    them after synchronisation."""

    def __init__(self, pairs: int = 512):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._pairs = []
        for _ in range(pairs):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(a)) or self._hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self._pairs.append((a, b))
        self._next = 0

    def arm(self) -> int:
        """Attach the next free pair to the next library call; returns its id."""
        if self._next >= len(self._pairs):
            raise RuntimeError("CallTimer: no free event pair (reset() first)")
        k = self._next
        self._next += 1
        a, b = self._pairs[k]
        _check(load_library().ddp_time_next_call(a, b), "ddp_time_next_call")
        return k

    def elapsed_ms(self, k: int) -> float:
        a, b = self._pairs[k]
        if self._hip.hipEventSynchronize(b):
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), a, b):
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def reset(self) -> None:
        self._next = 0

    def __del__(self):
        for a, b in getattr(self, "_pairs", []):
            self._hip.hipEventDestroy(a)
            self._hip.hipEventDestroy(b)


# ---------------------------------------------------------------------------
# Bucket plan
# ---------------------------------------------------------------------------

class Plan:
    """Owner of a ddp_plan handle (host) and, after upload(), its device table."""

    def __init__(self, handle: int, elem_bytes: int):
        self._h = ctypes.c_void_p(handle)
        self.elem_bytes = elem_bytes
        self._table = None
        self._segments = None
        self._numels = None

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value and _lib is not None:
            _lib.ddp_plan_free(self._h)
            self._h = ctypes.c_void_p(0)

    @property
    def handle(self):
        return self._h

    @property
    def num_params(self) -> int:
        return load_library().ddp_plan_num_params(self._h)

    @property
    def num_buckets(self) -> int:
        return load_library().ddp_plan_num_buckets(self._h)

    def bucket_numel(self, b: int) -> int:
        return load_library().ddp_plan_bucket_numel(self._h, b)

    def bucket_params(self, b: int) -> List[int]:
        L = load_library()
        k = L.ddp_plan_bucket_size(self._h, b)
        if k < 0:
            raise IndexError(b)
        out = (ctypes.c_int32 * max(k, 1))()
        _check(L.ddp_plan_bucket_params(self._h, b, out), "ddp_plan_bucket_params")
        return list(out[:k])

    def buckets(self) -> List[List[int]]:
        return [self.bucket_params(b) for b in range(self.num_buckets)]

    def param_bucket(self, i: int) -> int:
        return load_library().ddp_plan_param_bucket(self._h, i)

    def param_offset(self, i: int) -> int:
        return load_library().ddp_plan_param_offset(self._h, i)

    def param_numels(self) -> Tuple[int, ...]:
        """Element count of every parameter, in registration order."""
        if self._numels is None:
            L = load_library()
            self._numels = tuple(L.ddp_plan_param_numel(self._h, i)
                                 for i in range(self.num_params))
        return self._numels

    def device_bytes(self) -> int:
        return load_library().ddp_plan_device_bytes(self._h)

    def segment_bytes(self, p: int) -> int:
        return load_library().ddp_plan_segment_bytes(self._h, p)

    # A re-upload replaces a device table that kernels already enqueued may
    # still read, possibly on other streams (the reducer's communication
    # stream): the old table is released only after the device has drained.
    # The new table is kept only once the library has accepted it, so a
    # refused upload leaves the plan's previous table in place and alive.
    @staticmethod
    def _retire(old) -> None:
        if old is not None:
            import torch

            torch.cuda.synchronize(old.device)

    def upload_segments(self, p: int, device="cuda", stream=None) -> "Plan":
        """Upload the descriptor table ddp_allreduce_bucket needs for p ranks."""
        import torch

        nbytes = self.segment_bytes(p)
        fresh = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        _check(load_library().ddp_plan_upload_segments(
            self._h, p, _device_ptr(fresh), nbytes, _stream(stream)),
            "ddp_plan_upload_segments")
        self._retire(self._segments)
        self._segments = fresh
        return self

    def upload(self, device="cuda", stream=None) -> "Plan":
        import torch

        nbytes = self.device_bytes()
        fresh = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        _check(load_library().ddp_plan_upload(self._h, _device_ptr(fresh), nbytes,
                                              _stream(stream)), "ddp_plan_upload")
        self._retire(self._table)
        self._table = fresh
        return self


def ddp_bucket_plan(numel: Sequence[int], elem_bytes: int = 4,
                    bucket_cap_bytes: int = 25 * 1024 * 1024,
                    first_bucket_cap_bytes: int = 1024 * 1024,
                    order: Optional[Sequence[int]] = None) -> Plan:
    """Gradient buckets: reverse registration order, or `order` (the order in
    which gradients became ready, for the rebuild)."""
    L = load_library()
    n = len(numel)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in numel])
    out = ctypes.c_void_p()
    if order is None:
        _check(L.ddp_bucket_plan(arr, n, elem_bytes, bucket_cap_bytes, first_bucket_cap_bytes,
                                 ctypes.byref(out)), "ddp_bucket_plan")
    else:
        walk = (ctypes.c_int32 * max(len(order), 1))(*[int(v) for v in order])
        if len(order) != n:
            raise ValueError("order must list every parameter once")
        _check(L.ddp_bucket_plan_ordered(arr, n, walk, elem_bytes, bucket_cap_bytes,
                                         first_bucket_cap_bytes, ctypes.byref(out)),
               "ddp_bucket_plan_ordered")
    return Plan(out.value, elem_bytes)


BROADCAST_BUCKET_BYTES = 250 * 1024 * 1024


def ddp_coalesce_plan(numel: Sequence[int], elem_bytes: int,
                      cap_bytes: int = BROADCAST_BUCKET_BYTES) -> Plan:
    """Buckets of a coalesced broadcast (list order, none past the cap)."""
    L = load_library()
    n = len(numel)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in numel])
    out = ctypes.c_void_p()
    _check(L.ddp_coalesce_plan(arr, n, elem_bytes, cap_bytes, ctypes.byref(out)),
           "ddp_coalesce_plan")
    return Plan(out.value, elem_bytes)


def ddp_broadcast_coalesced(plan: Plan, tensor_table, p: int, root: int = 0,
                            stream=None) -> CommStats:
    """Broadcast every tensor of an uploaded coalesce plan from `root`;
    tensor_table is grad_pointer_table(tensors_per_rank)."""
    _check_grad_table(tensor_table, plan, p, "ddp_broadcast_coalesced")
    st = CommStats()
    _check(load_library().ddp_broadcast_coalesced(
        plan.handle, p, _device_ptr(tensor_table) if tensor_table is not None else None, root,
        _stream(stream), ctypes.byref(st)), "ddp_broadcast_coalesced")
    return st


def broadcast_coalesced(tensors: Sequence[Sequence], root: int = 0,
                        cap_bytes: int = BROADCAST_BUCKET_BYTES, stream=None):
    """tensors[r][i] = rank r's copy of tensor i (contiguous device tensors).
    Tensors are grouped by element size (one coalesced broadcast per group,
    as flattening needs one element type), bucketed in list order and
    broadcast from `root`. Returns the per-group stats."""
    p = len(tensors)
    n_t = len(tensors[0]) if p else 0
    groups = {}
    for i in range(n_t):
        groups.setdefault(tensors[0][i].element_size(), []).append(i)
    out = []
    for eb, idx in sorted(groups.items()):
        plan = ddp_coalesce_plan([tensors[0][i].numel() for i in idx], eb, cap_bytes)
        plan.upload(tensors[0][idx[0]].device, stream)
        table = grad_pointer_table([[tensors[r][i] for i in idx] for r in range(p)],
                                   tensors[0][idx[0]].device)
        out.append(ddp_broadcast_coalesced(plan, table, p, root, stream))
        if stream is not None:
            # allocated on the current stream, used on `stream`: keep the
            # memory from being reused before the kernels there have run
            plan._table.record_stream(stream)
            table.record_stream(stream)
    return out


def sync_module_states(params: Sequence[Sequence], buffers: Sequence[Sequence] = (),
                       root: int = 0, stream=None):
    """Make every rank's parameters and buffers equal to the root's: the
    init-time broadcast of parameters and buffers, coalesced (params[r][i],
    buffers[r][j] = rank r's copies)."""
    p = len(params)
    rows = [list(params[r]) + (list(buffers[r]) if buffers else []) for r in range(p)]
    return broadcast_coalesced(rows, root, BROADCAST_BUCKET_BYTES, stream)


def grad_pointer_table(grads: Sequence[Sequence], device="cuda"):
    """Device int64 tensor of p * n_params gradient addresses, rank-major.
    grads[r][i] is rank r's gradient of parameter i: contiguous device
    tensors of one element size, and the same element count for a parameter
    on every rank."""
    import torch

    if not grads:
        raise ValueError("grad_pointer_table needs at least one rank")
    first = grads[0]
    for r, rank in enumerate(grads):
        if len(rank) != len(first):
            raise ValueError(f"rank {r} has {len(rank)} gradients, rank 0 {len(first)}")
        for i, g in enumerate(rank):
            if (not g.is_contiguous() or g.element_size() != first[0].element_size()
                    or g.numel() != first[i].numel()):
                raise ValueError(f"gradient {i} of rank {r}: contiguous tensors of one element "
                                 "size and the same size on every rank are required")
    flat = [_device_ptr(g) for rank in grads for g in rank]
    _reject_overlaps(grads, flat)
    table = torch.tensor(flat, dtype=torch.int64, device=device)
    # what the table was built from, checked against the plan and the rank
    # count of every call that takes it (the kernels trust the addresses)
    table._ddp_ranks = len(grads)
    table._ddp_numel = tuple(g.numel() for g in first)
    table._ddp_elem_bytes = first[0].element_size() if first else 0
    return table


def _reject_overlaps(grads: Sequence[Sequence], addrs: Sequence[int]) -> None:
    """Every gradient of every rank must own its bytes: the kernels write each
    one, and two that share memory would race."""
    import numpy as np

    if not addrs:
        return
    nbytes = np.array([g.numel() * g.element_size() for rank in grads for g in rank],
                      dtype=np.int64)
    start = np.array(addrs, dtype=np.int64)
    live = np.nonzero(nbytes > 0)[0]
    if live.size < 2:
        return
    order = live[np.argsort(start[live], kind="stable")]
    ends = start[order] + nbytes[order]
    clash = np.nonzero(start[order][1:] < ends[:-1])[0]
    if clash.size:
        n_params = len(grads[0])
        a, b = (int(order[clash[0]]), int(order[clash[0] + 1]))
        raise ValueError(f"gradient {a % n_params} of rank {a // n_params} and gradient "
                         f"{b % n_params} of rank {b // n_params} share memory")


def _check_grad_table(table, plan: "Plan", p: int, what: str) -> None:
    """The table must have been built by grad_pointer_table for p ranks of
    tensors shaped as the plan's parameters: the kernels read p * n_params
    addresses from it and write every element of every one."""
    import torch

    if table is None:
        return  # the library refuses a NULL table wherever it would be read
    if not isinstance(table, torch.Tensor) or getattr(table, "_ddp_numel", None) is None:
        raise TypeError(f"{what}: build the gradient table with grad_pointer_table")
    if table.dtype != torch.int64 or not table.is_contiguous():
        raise TypeError(f"{what}: the gradient table must be a contiguous int64 tensor")
    if table._ddp_ranks != p or table.numel() != p * plan.num_params:
        raise ValueError(f"{what}: the gradient table holds {table._ddp_ranks} ranks of "
                         f"{len(table._ddp_numel)} tensors; the call needs {p} ranks of "
                         f"{plan.num_params}")
    if table._ddp_elem_bytes != plan.elem_bytes and plan.num_params > 0:
        raise ValueError(f"{what}: the gradients have {table._ddp_elem_bytes}-byte elements, "
                         f"the plan {plan.elem_bytes}")
    want = plan.param_numels()
    if table._ddp_numel != want:
        i = next(k for k, (a, b) in enumerate(zip(table._ddp_numel, want)) if a != b)
        raise ValueError(f"{what}: tensor {i} has {table._ddp_numel[i]} elements, the plan "
                         f"{want[i]}")
    _device_ptr(table)


def _check_bucket_bufs(plan: "Plan", bucket: int, bufs: Sequence, what: str) -> None:
    """Flat bucket buffers: one per rank, each exactly the bucket's elements,
    contiguous, of the plan's element size."""
    if not bufs:
        raise ValueError(f"{what}: needs one bucket buffer per rank")
    n = plan.bucket_numel(bucket)
    if n < 0:
        return  # bucket out of range: the library reports it
    for r, t in enumerate(bufs):
        if (t.numel() != n or t.dtype != bufs[0].dtype or not t.is_contiguous()
                or t.element_size() != plan.elem_bytes):
            raise ValueError(f"{what}: bucket buffer of rank {r} must be a contiguous tensor of "
                             f"{n} elements of {plan.elem_bytes} bytes (got {t.numel()} of "
                             f"{t.element_size()})")


def ddp_flatten(plan: Plan, bucket: int, grad_table, bucket_bufs: Sequence,
                prescale_divisor: float = 1.0, stream=None) -> None:
    p = len(bucket_bufs)
    _check_bucket_bufs(plan, bucket, bucket_bufs, "ddp_flatten")
    _check_grad_table(grad_table, plan, p, "ddp_flatten")
    _check(load_library().ddp_flatten(plan.handle, bucket, p, _device_ptr(grad_table),
                                      _ptrs(bucket_bufs), _dtype_code(bucket_bufs[0]),
                                      float(prescale_divisor), _stream(stream)),
           "ddp_flatten")


def ddp_unflatten(plan: Plan, bucket: int, bucket_bufs: Sequence, grad_table,
                  stream=None) -> None:
    p = len(bucket_bufs)
    _check_bucket_bufs(plan, bucket, bucket_bufs, "ddp_unflatten")
    _check_grad_table(grad_table, plan, p, "ddp_unflatten")
    _check(load_library().ddp_unflatten(plan.handle, bucket, p, _ptrs(bucket_bufs),
                                        _device_ptr(grad_table), _dtype_code(bucket_bufs[0]),
                                        _stream(stream)), "ddp_unflatten")


def ddp_allreduce_bucket(plan: Plan, bucket: int, grad_table, p: int, dtype=None,
                         avg: str = "none", tokens=None, stream=None) -> CommStats:
    """Flatten + ring all-reduce + unflatten of one bucket, in one pass."""
    import torch

    if dtype is None:
        dtype = torch.float32 if plan.elem_bytes == 4 else torch.bfloat16
    code = DTYPE_F32 if dtype == torch.float32 else DTYPE_BF16
    _check_grad_table(grad_table, plan, p, "ddp_allreduce_bucket")
    st = CommStats()
    _check(load_library().ddp_allreduce_bucket(
        plan.handle, bucket, p, _device_ptr(grad_table), code, AVG[avg], _tokens(tokens, p),
        _stream(stream), ctypes.byref(st)), "ddp_allreduce_bucket")
    return st


def ddp_allreduce_buckets(plan: Plan, first_bucket: int, n_buckets: int, grad_table, p: int,
                          dtype=None, avg: str = "none", tokens=None, stream=None) -> CommStats:
    """ddp_allreduce_bucket for a run of consecutive buckets, one launch."""
    import torch

    if dtype is None:
        dtype = torch.float32 if plan.elem_bytes == 4 else torch.bfloat16
    code = DTYPE_F32 if dtype == torch.float32 else DTYPE_BF16
    _check_grad_table(grad_table, plan, p, "ddp_allreduce_buckets")
    st = CommStats()
    _check(load_library().ddp_allreduce_buckets(
        plan.handle, first_bucket, n_buckets, p, _device_ptr(grad_table), code, AVG[avg],
        _tokens(tokens, p), _stream(stream), ctypes.byref(st)), "ddp_allreduce_buckets")
    return st


class Reducer:
    """Owner of a ddp_reducer: bucket all-reduces launched on `comm_stream`
    as parameters are marked ready (see include/ddpsim.h)."""

    def __init__(self, plan: Plan, p: int, grad_table, dtype=None, avg: str = "none",
                 tokens=None, comm_stream=None):
        import torch

        if dtype is None:
            dtype = torch.float32 if plan.elem_bytes == 4 else torch.bfloat16
        code = DTYPE_F32 if dtype == torch.float32 else DTYPE_BF16
        _check_grad_table(grad_table, plan, p, "Reducer")
        self._plan, self._table = plan, grad_table  # kept alive
        self._h = ctypes.c_void_p()
        self.comm_stream = comm_stream if comm_stream is not None else torch.cuda.current_stream()
        _check(load_library().ddp_reducer_create(
            plan.handle, p, _device_ptr(grad_table) if grad_table is not None else None, code,
            AVG[avg], _tokens(tokens, p), _stream(self.comm_stream), ctypes.byref(self._h)),
            "ddp_reducer_create")

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value and _lib is not None:
            _lib.ddp_reducer_free(self._h)
            self._h = ctypes.c_void_p(0)

    def prepare(self) -> None:
        _check(load_library().ddp_reducer_prepare(self._h), "ddp_reducer_prepare")

    def mark_ready(self, param: int, event=None) -> None:
        """event: a torch.cuda.Event recorded after the gradients were written."""
        handle = event.cuda_event if event is not None else None
        _check(load_library().ddp_reducer_mark_ready(self._h, param, handle),
               "ddp_reducer_mark_ready")

    def finalize(self, wait_stream=None) -> None:
        _check(load_library().ddp_reducer_finalize(self._h, _stream(wait_stream)),
               "ddp_reducer_finalize")

    def set_max_workgroups(self, n: int) -> None:
        """Cap each all-reduce launch at n workgroups (0: one per tile)."""
        _check(load_library().ddp_reducer_set_max_workgroups(self._h, n),
               "ddp_reducer_set_max_workgroups")

    def ready_order(self) -> List[int]:
        """Parameters in the order they were marked ready this (or the last)
        pass: the order to rebuild the buckets from."""
        L = load_library()
        n = L.ddp_reducer_ready_order(self._h, None, 0)
        a = (ctypes.c_int32 * max(n, 1))()
        L.ddp_reducer_ready_order(self._h, a, n)
        return list(a[:n])

    def launch_log(self):
        L = load_library()
        n = L.ddp_reducer_launch_log(self._h, None, None, None, 0)
        a = (ctypes.c_int32 * max(n, 1))()
        b = (ctypes.c_int32 * max(n, 1))()
        c = (ctypes.c_int32 * max(n, 1))()
        L.ddp_reducer_launch_log(self._h, a, b, c, n)
        return [(a[k], b[k], c[k]) for k in range(n)]


# ---------------------------------------------------------------------------
# Collectives
# ---------------------------------------------------------------------------

def ring_allreduce_sim_workspace(p: int, n: int, dtype: int, algo: str = "fused") -> int:
    return load_library().ring_allreduce_sim_workspace(p, n, dtype, ALGO[algo])


def ring_allreduce_sim(bufs: Sequence, avg: str = "none", tokens=None,
                       algo: str = "fused", workspace=None, stream=None) -> CommStats:
    p = len(bufs)
    n = _numel_all(bufs)
    st = CommStats()
    ws_ptr = _device_ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().ring_allreduce_sim(
        _ptrs(bufs), p, n, _dtype_code(bufs[0]), AVG[avg], _tokens(tokens, p),
        ALGO[algo], ws_ptr, ws_bytes, _stream(stream), ctypes.byref(st)),
        "ring_allreduce_sim")
    return st


NOALLOC_SCRATCH_BYTES = 64 << 20  # DDP_NOALLOC_SCRATCH_BYTES


def ring_allreduce_sim_noalloc(bufs: Sequence, avg: str = "none", tokens=None,
                               algo: str = "fused", stream=None) -> CommStats:
    """ring_allreduce_sim without a workspace argument: the bf16 ring's
    workspace is the library's per-GPU scratch array (at most
    NOALLOC_SCRATCH_BYTES); nothing is allocated."""
    p = len(bufs)
    n = _numel_all(bufs)
    st = CommStats()
    _check(load_library().ring_allreduce_sim_noalloc(
        _ptrs(bufs), p, n, _dtype_code(bufs[0]), AVG[avg], _tokens(tokens, p), ALGO[algo],
        _stream(stream), ctypes.byref(st)), "ring_allreduce_sim_noalloc")
    return st


def ring_allreduce_sim_steps(bufs: Sequence, first_step: int, n_steps: int,
                             avg: str = "none", tokens=None, stream=None) -> None:
    p = len(bufs)
    n = _numel_all(bufs)
    if _dtype_code(bufs[0]) != DTYPE_F32:
        raise TypeError("ring_allreduce_sim_steps runs on float32 buffers")
    _check(load_library().ring_allreduce_sim_steps(
        _ptrs(bufs), p, n, AVG[avg], _tokens(tokens, p), first_step, n_steps,
        _stream(stream)), "ring_allreduce_sim_steps")


def allreduce_sim_workspace(p: int, n: int, dtype: int, schedule: str = "ring",
                            steps: bool = False) -> int:
    return load_library().allreduce_sim_workspace(p, n, dtype, SCHEDULES[schedule],
                                                  1 if steps else 0)


def allreduce_sim(bufs: Sequence, schedule: str = "ring", steps: bool = False,
                  avg: str = "none", tokens=None, workspace=None, stream=None) -> CommStats:
    """In-place all-reduce under a schedule ("ring", "recursive_doubling",
    "rabenseifner", "tree"), as one fused pass or step by step."""
    p = len(bufs)
    n = _numel_all(bufs)
    st = CommStats()
    ws_ptr = _device_ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().allreduce_sim(
        _ptrs(bufs), p, n, _dtype_code(bufs[0]), AVG[avg], _tokens(tokens, p),
        SCHEDULES[schedule], 1 if steps else 0, ws_ptr, ws_bytes, _stream(stream),
        ctypes.byref(st)), "allreduce_sim")
    return st


def schedule_time(schedule: str, p: int, nbytes: float, alpha: float, beta: float) -> float:
    """Latency-bandwidth model time of one all-reduce of nbytes."""
    return load_library().ddp_schedule_time(SCHEDULES[schedule], p, nbytes, alpha, beta)


def choose_schedule(p: int, nbytes: int, alpha: float, beta: float,
                    candidates: Sequence[str] = ("ring", "recursive_doubling")) -> str:
    """The candidate schedule with the smallest model time (ties to the lower
    schedule number)."""
    mask = 0
    for c in candidates:
        mask |= 1 << SCHEDULES[c]
    s = load_library().ddp_choose_schedule(p, nbytes, alpha, beta, mask)
    if s < 0:
        raise DDPError(1, "ddp_choose_schedule",
                       load_library().ddp_last_error().decode(errors="replace"))
    return {v: k for k, v in SCHEDULES.items()}[s]


def overlap_step_time(plan: "Plan", ready: Sequence[float],
                      bucket_time: Sequence[float]) -> Tuple[float, float]:
    """(step, exposed) seconds of a backward whose bucket all-reduces overlap
    it: ready[i] is parameter i's ready time, bucket_time[b] bucket b's
    all-reduce duration."""
    if len(ready) != plan.num_params or len(bucket_time) != plan.num_buckets:
        raise ValueError(f"overlap_step_time: {plan.num_params} ready times and "
                         f"{plan.num_buckets} bucket times expected, got {len(ready)} "
                         f"and {len(bucket_time)}")
    rd = (ctypes.c_double * max(1, len(ready)))(*ready)
    bt = (ctypes.c_double * max(1, len(bucket_time)))(*bucket_time)
    step, exposed = ctypes.c_double(), ctypes.c_double()
    _check(load_library().ddp_overlap_step_time(plan.handle, rd, bt, ctypes.byref(step),
                                                ctypes.byref(exposed)),
           "ddp_overlap_step_time")
    return step.value, exposed.value


def reduce_scatter_sim(inputs: Sequence, outputs: Sequence, avg: str = "none",
                       tokens=None, stream=None) -> CommStats:
    p = len(inputs)
    n = _numel_all(inputs)
    st = CommStats()
    _check(load_library().reduce_scatter_sim(
        _ptrs(inputs), _ptrs(outputs), p, n, _dtype_code(inputs[0]), AVG[avg],
        _tokens(tokens, p), _stream(stream), ctypes.byref(st)), "reduce_scatter_sim")
    return st


def allgather_sim(inputs: Sequence, outputs: Sequence, stream=None) -> CommStats:
    p = len(outputs)
    n = _numel_all(outputs)
    st = CommStats()
    _check(load_library().allgather_sim(
        _ptrs(inputs), _ptrs(outputs), p, n, _dtype_code(outputs[0]), _stream(stream),
        ctypes.byref(st)), "allgather_sim")
    return st


def broadcast_sim(bufs: Sequence, src: int = 0, stream=None) -> CommStats:
    p = len(bufs)
    n = _numel_all(bufs)
    st = CommStats()
    _check(load_library().broadcast_sim(
        _ptrs(bufs), p, n, src, _dtype_code(bufs[0]), _stream(stream), ctypes.byref(st)),
        "broadcast_sim")
    return st
