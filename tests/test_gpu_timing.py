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
