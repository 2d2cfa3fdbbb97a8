"""GPU parity for the reducer: gradients produced on one stream in some
order, each marked ready with an event; bucket all-reduces launched on a
second stream. The final gradients must equal the oracle's flatten -> ring
-> unflatten bit for bit, and the launch runs must equal the oracle's
schedule for the same mark order."""
import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from helpers import assert_bits_equal, make_grads, to_dev, to_host, tokens_for

pytestmark = pytest.mark.gpu

SIZES = [5000, 0, 7, 4096, 4097, 1, 33_333, 12, 0, 65_536 + 9, 3, 100_000]


def _oracle_sync(oracle, host, sizes, eb, cap, first, avg, tokens):
    p = len(host)
    oplan = oracle.bucket_plan(sizes, eb, cap, first)
    want = [[g.copy() for g in rank] for rank in host]
    for b in range(oplan.num_buckets):
        flats = [oracle.flatten(want[r], oplan, b) for r in range(p)]
        red, _ = oracle.ring_allreduce(flats, avg=avg, tokens=tokens, want_log=False)
        for r in range(p):
            oracle.unflatten(red[r], oplan, b, want[r])
    return want, oplan


@pytest.mark.parametrize("order_kind", ["reverse", "forward", "random"])
@pytest.mark.parametrize("bf16,avg", [(False, "world"), (True, "tokens")])
def test_reducer_overlapped_sync(oracle, order_kind, bf16, avg):
    p = 4
    eb = 2 if bf16 else 4
    cap, first = 96 * 1024, 8 * 1024
    plan = ddp.ddp_bucket_plan(SIZES, eb, cap, first).upload_segments(p)
    host, grads = make_grads(p, SIZES, 1100, bf16, oracle, "aligned")
    sources = [[to_dev(host[r][i]) for i in range(len(SIZES))] for r in range(p)]
    for r in range(p):
        for g in grads[r]:
            g.zero_()
    table = ddp.grad_pointer_table(grads)
    tokens = tokens_for(p, 5) if avg == "tokens" else None
    comm = torch.cuda.Stream()
    producer = torch.cuda.Stream()
    torch.cuda.synchronize()
    red = ddp.Reducer(plan, p, table, avg=avg, tokens=tokens, comm_stream=comm)
    order = list(range(len(SIZES)))
    if order_kind == "reverse":
        order = order[::-1]
    elif order_kind == "random":
        order = [int(i) for i in np.random.default_rng(7).permutation(len(SIZES))]
    events = []
    red.prepare()
    with torch.cuda.stream(producer):
        for i in order:
            for r in range(p):
                grads[r][i].copy_(sources[r][i])  # the "backward" writes grad i
            ev = torch.cuda.Event()
            ev.record(producer)
            events.append(ev)
            red.mark_ready(i, ev)
    red.finalize(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want, oplan = _oracle_sync(oracle, host, SIZES, eb, cap, first, avg, tokens)
    for r in range(p):
        for i in range(len(SIZES)):
            assert_bits_equal(to_host(grads[r][i]), want[r][i], f"rank {r} param {i}")
    runs, total = oracle.reducer_schedule(oplan, order)
    assert red.launch_log() == runs and total == plan.num_buckets


def test_reducer_second_pass_and_unready_bucket(oracle):
    p = 2
    plan = ddp.ddp_bucket_plan(SIZES, 4, 96 * 1024, 8 * 1024).upload_segments(p)
    host, grads = make_grads(p, SIZES, 1200, False, oracle, "aligned")
    table = ddp.grad_pointer_table(grads)
    red = ddp.Reducer(plan, p, table, avg="none")
    # a pass that leaves the last bucket's parameter unmarked
    red.prepare()
    skip = plan.bucket_params(plan.num_buckets - 1)[-1]
    for i in reversed(range(len(SIZES))):
        if i != skip:
            red.mark_ready(i)
    with pytest.raises(ddp.DDPError, match="ENOTREADY"):
        red.finalize()
    # a complete pass afterwards works and sums the (partly reduced) values
    red.prepare()
    for i in reversed(range(len(SIZES))):
        red.mark_ready(i)
    red.finalize()
    torch.cuda.synchronize()
    assert len(red.launch_log()) == plan.num_buckets


@pytest.mark.parametrize("cap", [1, 7, 300])
def test_capped_workgroups_give_the_same_bits(oracle, cap):
    """A reducer whose launches are capped at `cap` workgroups walks the
    tiles grid-stride: same results as the oracle."""
    p = 4
    eb, cap_b, first = 4, 96 * 1024, 8 * 1024
    plan = ddp.ddp_bucket_plan(SIZES, eb, cap_b, first).upload_segments(p)
    host, grads = make_grads(p, SIZES, 1400 + cap, False, oracle, "mixed")
    table = ddp.grad_pointer_table(grads)
    red = ddp.Reducer(plan, p, table, avg="world")
    red.set_max_workgroups(cap)
    red.prepare()
    for i in reversed(range(len(SIZES))):
        red.mark_ready(i)
    red.finalize()
    torch.cuda.synchronize()
    want, _ = _oracle_sync(oracle, host, SIZES, eb, cap_b, first, "world", None)
    for r in range(p):
        for i in range(len(SIZES)):
            assert_bits_equal(to_host(grads[r][i]), want[r][i], f"cap {cap} rank {r} param {i}")
