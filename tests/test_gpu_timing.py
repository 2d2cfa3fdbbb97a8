"""ddp_time_next_call: the events bracket exactly the next call's kernels
and are consumed by it."""
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_events_time_the_next_call_only():
    p, n = 8, 1 << 22
    bufs = [W.normal_torch(n, 1.0, 1, r, "cuda") for r in range(p)]
    timer = ddp.CallTimer(pairs=4)
    k0 = timer.arm()
    ddp.ring_allreduce_sim(bufs, avg="world")          # timed: one kernel
    k1 = timer.arm()
    ddp.ring_allreduce_sim(bufs, avg="world", algo="ring")  # timed: 14 kernels
    ddp.ring_allreduce_sim(bufs, avg="world")          # not timed
    torch.cuda.synchronize()
    fused, ring = timer.elapsed_ms(k0), timer.elapsed_ms(k1)
    assert 0 < fused < ring
    # a failed call consumes the request too (nothing recorded, no error later)
    timer.arm()
    with pytest.raises(ddp.DDPError):
        ddp.ring_allreduce_sim(bufs[:1] + bufs[:1], avg="world")  # aliasing buffers
    ddp.ring_allreduce_sim(bufs, avg="world")
    torch.cuda.synchronize()


def test_host_only_calls_leave_the_request_pending():
    """Planning, the models and plan uploads launch nothing, so the armed
    events go to the next call that does launch kernels."""
    p, sizes = 4, [5000, 70_000, 123]
    plan = ddp.ddp_bucket_plan(sizes, 4, 64 * 1024, 8 * 1024)
    grads = [[W.normal_torch(n, 1.0, 2, r, "cuda", stream=i) for i, n in enumerate(sizes)]
             for r in range(p)]
    table = ddp.grad_pointer_table(grads)
    timer = ddp.CallTimer(pairs=2)
    k = timer.arm()
    ddp.ddp_bucket_plan(sizes, 4, 64 * 1024, 8 * 1024)
    ddp.schedule_time("ring", p, 1e6, 1e-5, 1 / 50e9)
    ddp.choose_schedule(p, 10 ** 6, 1e-5, 1 / 50e9)
    ddp.overlap_step_time(plan, [0.0] * len(sizes), [0.0] * plan.num_buckets)
    plan.upload_segments(p)
    ddp.ddp_allreduce_buckets(plan, 0, plan.num_buckets, table, p, avg="world")
    torch.cuda.synchronize()
    assert timer.elapsed_ms(k) > 0
