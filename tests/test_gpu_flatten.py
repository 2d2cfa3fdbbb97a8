"""GPU parity: flatten / unflatten through the plan against the oracle, and
the bucketed path end to end (flatten -> all-reduce -> unflatten) on small
gradient sets, including gradients at unaligned addresses, zero-size
parameters, pre-division and bf16."""
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def _grads(p, sizes, seed, bf16, oracle, misalign):
    """Per-rank gradients as views into one arena per rank; with misalign the
    views start at odd element offsets."""
    host = [[W.normal_np(n, 1.0, seed, r, stream=i) for i, n in enumerate(sizes)]
            for r in range(p)]
    if bf16:
        host = [[oracle.f32_to_bf16(g) for g in rank] for rank in host]
    dt = torch.bfloat16 if bf16 else torch.float32
    grads = []
    for r in range(p):
        total = sum(sizes) + 3 * len(sizes) + 8
        arena = torch.zeros(total, dtype=dt, device="cuda")
        off = 1 if misalign else 0
        views = []
        for i, n in enumerate(sizes):
            if not misalign:
                off = (off + 7) // 8 * 8
            v = arena[off:off + n]
            v.copy_(to_dev(host[r][i]))
            views.append(v)
            off += n + (1 if misalign else 0)
        grads.append(views)
    return host, grads


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("prescale", [1.0, 4.0, 3.0])
def test_flatten_unflatten(oracle, bf16, misalign, prescale):
    p = 3
    sizes = [5000, 0, 7, 4096, 4097, 1, 33_333, 12, 0, 65_536 + 9]
    eb = 2 if bf16 else 4
    cap, first = 64 * 1024, 4 * 1024
    plan = ddp.ddp_bucket_plan(sizes, eb, cap, first).upload()
    oplan = oracle.bucket_plan(sizes, eb, cap, first)
    host, grads = _grads(p, sizes, 700, bf16, oracle, misalign)
    table = ddp.grad_pointer_table(grads)
    dt = torch.bfloat16 if bf16 else torch.float32
    for b in range(plan.num_buckets):
        nb = plan.bucket_numel(b)
        bufs = [torch.empty(nb, dtype=dt, device="cuda") for _ in range(p)]
        ddp.ddp_flatten(plan, b, table, bufs, prescale_divisor=prescale)
        torch.cuda.synchronize()
        for r in range(p):
            want = oracle.flatten(host[r], oplan, b, divisor=prescale)
            assert_bits_equal(to_host(bufs[r]), want, f"bucket {b} rank {r}")
        # unflatten writes the bucket back over the gradients
        for buf in bufs:
            buf.mul_(-1)
        ddp.ddp_unflatten(plan, b, bufs, table)
        torch.cuda.synchronize()
        for r in range(p):
            flat = to_host(bufs[r])
            for i in oplan.bucket_params(b):
                off = oplan.offset[i]
                assert_bits_equal(to_host(grads[r][i]), flat[off:off + sizes[i]], f"param {i}")


@pytest.mark.parametrize("p", [2, 8])
def test_bucketed_sync_end_to_end(oracle, p):
    sizes = [W.numel(s) for _, s in W.gpt2_small_params(n_layer=2, d=64, vocab=1000, ctx=128)]
    cap, first = 16 * 1024, 2 * 1024
    plan = ddp.ddp_bucket_plan(sizes, 4, cap, first).upload()
    oplan = oracle.bucket_plan(sizes, 4, cap, first)
    host, grads = _grads(p, sizes, 800, False, oracle, False)
    table = ddp.grad_pointer_table(grads)
    want = [[g.copy() for g in rank] for rank in host]
    for b in range(plan.num_buckets):
        bufs = [torch.empty(plan.bucket_numel(b), device="cuda") for _ in range(p)]
        ddp.ddp_flatten(plan, b, table, bufs)
        ddp.ring_allreduce_sim(bufs, avg="world")
        ddp.ddp_unflatten(plan, b, bufs, table)
        flats = [oracle.flatten(want[r], oplan, b) for r in range(p)]
        red, _ = oracle.ring_allreduce(flats, avg="world", want_log=False)
        for r in range(p):
            oracle.unflatten(red[r], oplan, b, want[r])
    torch.cuda.synchronize()
    for r in range(p):
        for i in range(len(sizes)):
            assert_bits_equal(to_host(grads[r][i]), want[r][i], f"rank {r} param {i}")


def test_flatten_errors():
    import ctypes

    plan = ddp.ddp_bucket_plan([10, 20], 4, 100, 40)
    assert plan.bucket_numel(0) == 20
    bufs = [torch.empty(20, device="cuda") for _ in range(2)]
    grads = [[torch.zeros(n, device="cuda") for n in (10, 20)] for _ in range(2)]
    table = ddp.grad_pointer_table(grads)
    with pytest.raises(ddp.DDPError, match="ENOTREADY"):
        ddp.ddp_flatten(plan, 0, table, bufs)
    plan.upload()
    with pytest.raises(ddp.DDPError, match="ERANGE"):
        ddp.ddp_flatten(plan, 5, table, bufs)
    # the binding refuses buffers of the wrong element size or length ...
    with pytest.raises(ValueError, match="rank 0"):
        ddp.ddp_flatten(plan, 0, table, [b.to(torch.bfloat16) for b in bufs])
    with pytest.raises(ValueError, match="rank 1"):
        ddp.ddp_unflatten(plan, 0, [bufs[0], bufs[1][:19]], table)
    # ... and the library refuses a dtype the plan was not built for
    L = ddp.load_library()
    ptrs = (ctypes.c_void_p * 2)(*[b.data_ptr() for b in bufs])
    assert L.ddp_flatten(plan.handle, 0, 2, table.data_ptr(), ptrs, 1, 1.0, None) == 1
