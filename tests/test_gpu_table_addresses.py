"""GPU parity with the device pointer tables placed where bit 31 of their
address is set, and where it is clear.

Kernels read a 64-bit rank address from a table whose own address they
assemble from two 32-bit halves (lane reads return signed 32-bit values); a
low half that is sign-extended instead of zero-extended corrupts the
address exactly when bit 31 is set. Where torch happens to allocate a table
decides which case a test meets, so these tests place copies of the tables
at both kinds of address on purpose and compare every result with the
oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from helpers import assert_bits_equal, make_grads, to_host

pytestmark = pytest.mark.gpu

SIZES = [5000, 7, 4096, 4097, 1, 33_333, 65_536 + 9, 100_000]


@pytest.fixture(scope="module")
def spare():
    """2 GiB + 1 MiB of device memory: every 2^31-aligned window boundary
    inside it flips bit 31 of the address."""
    buf = torch.empty(((1 << 31) + (1 << 20)) // 8, dtype=torch.int64, device="cuda")
    yield buf
    del buf
    torch.cuda.synchronize()


def _table_at(spare, table, bit31):
    """A copy of `table` inside `spare`, at the first 256-byte aligned
    address whose bit 31 equals `bit31`; it carries the table's checks."""
    n = table.numel()
    base = spare.data_ptr()
    a = (base + 255) // 256 * 256
    if ((a >> 31) & 1) != bit31:
        a = ((a >> 31) + 1) << 31
    assert ((a >> 31) & 1) == bit31
    off = (a - base) // 8
    assert off + n <= spare.numel()
    view = spare[off:off + n]
    view.copy_(table)
    view._ddp_ranks = table._ddp_ranks
    view._ddp_numel = table._ddp_numel
    view._ddp_elem_bytes = table._ddp_elem_bytes
    assert (view.data_ptr() >> 31) & 1 == bit31
    return view


def _oracle_sync(oracle, host, sizes, eb, cap, first):
    p = len(host)
    oplan = oracle.bucket_plan(sizes, eb, cap, first)
    want = [[g.copy() for g in rank] for rank in host]
    for b in range(oplan.num_buckets):
        flats = [oracle.flatten(want[r], oplan, b) for r in range(p)]
        red, _ = oracle.ring_allreduce(flats, avg="world", tokens=None, want_log=False)
        for r in range(p):
            oracle.unflatten(red[r], oplan, b, want[r])
    return want


@pytest.mark.parametrize("bit31", [0, 1])
@pytest.mark.parametrize("layout", ["aligned", "odd"])
@pytest.mark.parametrize("p,root", [(8, 0), (8, 5), (64, 63)])
def test_coalesced_broadcast_table_address(oracle, spare, bit31, layout, p, root):
    host, views = make_grads(p, SIZES, 4100 + p + root, False, oracle, layout)
    host_t = [[h.copy() for h in rank] for rank in host]
    cap = 40_000 * 4
    plan = ddp.ddp_coalesce_plan(SIZES, 4, cap).upload()
    table = _table_at(spare, ddp.grad_pointer_table(views), bit31)
    ddp.ddp_broadcast_coalesced(plan, table, p, root)
    torch.cuda.synchronize()
    want, _, _ = oracle.broadcast_coalesced(host_t, root=root, cap_bytes=cap)
    for r in range(p):
        for i in range(len(SIZES)):
            got = to_host(views[r][i])
            assert np.array_equal(got.view(np.uint8), want[r][i].view(np.uint8)), (r, i)


@pytest.mark.parametrize("bit31", [0, 1])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("p", [8, 64])
def test_bucket_allreduce_table_address(oracle, spare, bit31, bf16, p):
    eb = 2 if bf16 else 4
    cap, first = 96 * 1024, 8 * 1024
    plan = ddp.ddp_bucket_plan(SIZES, eb, cap, first).upload_segments(p)
    host, grads = make_grads(p, SIZES, 4200 + p, bf16, oracle, "odd")
    table = _table_at(spare, ddp.grad_pointer_table(grads), bit31)
    ddp.ddp_allreduce_buckets(plan, 0, plan.num_buckets, table, p, avg="world")
    torch.cuda.synchronize()
    want = _oracle_sync(oracle, host, SIZES, eb, cap, first)
    for r in range(p):
        for i in range(len(SIZES)):
            assert_bits_equal(to_host(grads[r][i]), want[r][i], f"rank {r} param {i}")


@pytest.mark.parametrize("bit31", [0, 1])
def test_flatten_unflatten_table_address(oracle, spare, bit31):
    p, eb = 8, 4
    cap, first = 96 * 1024, 8 * 1024
    plan = ddp.ddp_bucket_plan(SIZES, eb, cap, first).upload()
    host, grads = make_grads(p, SIZES, 4300, False, oracle, "odd")
    table = _table_at(spare, ddp.grad_pointer_table(grads), bit31)
    oplan = oracle.bucket_plan(SIZES, eb, cap, first)
    for b in range(plan.num_buckets):
        bufs = [torch.empty(plan.bucket_numel(b), dtype=torch.float32, device="cuda")
                for _ in range(p)]
        ddp.ddp_flatten(plan, b, table, bufs)
        torch.cuda.synchronize()
        for r in range(p):
            assert_bits_equal(to_host(bufs[r]), oracle.flatten(host[r], oplan, b),
                              f"flatten bucket {b} rank {r}")
        for r in range(p):
            bufs[r].neg_()
        ddp.ddp_unflatten(plan, b, bufs, table)
        torch.cuda.synchronize()
        for r in range(p):
            back = [g.copy() for g in host[r]]
            oracle.unflatten(-oracle.flatten(host[r], oplan, b), oplan, b, back)
            for i in range(len(SIZES)):
                assert_bits_equal(to_host(grads[r][i]), back[i], f"unflatten b{b} r{r} p{i}")
            host[r] = back
