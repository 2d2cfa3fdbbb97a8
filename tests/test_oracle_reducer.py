"""Pins for the oracle's reducer schedule ("PyTorch DDP Deep Dive", Part 2
"Step 2: backward": pending counts per bucket, buckets launched in index
order, an out-of-turn bucket waits).

Besides hand cases, the state machine is checked against a closed form: the
bucket b is launched by the mark at which the last of buckets 0..b became
complete, i.e. launch_mark(b) = max over b' <= b of complete_mark(b')."""
import numpy as np
import pytest


def _plan(oracle, sizes, cap=64, first=16):
    return oracle.bucket_plan(sizes, 4, cap, first)


def test_reverse_registration_order_fires_each_bucket_at_its_last_param(oracle):
    sizes = [3, 5, 2, 8, 1, 4, 6, 7, 2, 9]
    plan = _plan(oracle, sizes)
    order = list(range(len(sizes)))[::-1]  # backward produces the last first
    runs, total = oracle.reducer_schedule(plan, order)
    assert total == plan.num_buckets
    want = []
    for b in range(plan.num_buckets):
        last = max(order.index(i) for i in plan.bucket_params(b))
        want.append((last, b, 1))
    assert runs == want


def test_forward_order_fires_everything_at_the_end(oracle):
    sizes = [3, 5, 2, 8, 1, 4, 6, 7, 2, 9]
    plan = _plan(oracle, sizes)
    runs, total = oracle.reducer_schedule(plan, list(range(len(sizes))))
    assert runs == [(len(sizes) - 1, 0, plan.num_buckets)]


@pytest.mark.parametrize("seed", range(30))
def test_random_orders_match_the_closed_form(oracle, seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 40))
    sizes = [int(v) for v in rng.integers(0, 20, size=P)]
    plan = _plan(oracle, sizes, cap=int(rng.integers(1, 80)), first=int(rng.integers(1, 40)))
    order = [int(i) for i in rng.permutation(P)]
    runs, total = oracle.reducer_schedule(plan, order)
    assert total == plan.num_buckets
    complete = [max(order.index(i) for i in plan.bucket_params(b)) for b in range(plan.num_buckets)]
    launch = [max(complete[:b + 1]) for b in range(plan.num_buckets)]
    got = {}
    for m, b0, k in runs:
        for b in range(b0, b0 + k):
            got[b] = m
    assert [got[b] for b in range(plan.num_buckets)] == launch
    # runs are consecutive and in order
    nxt = 0
    for _, b0, k in runs:
        assert b0 == nxt
        nxt += k


def test_incomplete_and_double_marks(oracle):
    sizes = [3, 5, 2, 8]
    plan = _plan(oracle, sizes, cap=16, first=8)
    assert plan.num_buckets >= 2
    # leave one parameter of bucket 0 unmarked: nothing can launch
    b0 = plan.bucket_params(0)
    order = [i for i in range(len(sizes)) if i != b0[0]]
    runs, total = oracle.reducer_schedule(plan, order)
    assert runs == [] and total == 0
    with pytest.raises(oracle.OracleError):
        oracle.reducer_schedule(plan, [3, 3])
    with pytest.raises(oracle.OracleError):
        oracle.reducer_schedule(plan, [7])
