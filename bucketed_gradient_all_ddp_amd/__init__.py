"""bucketed_gradient_all_ddp_amd -- the data-parallel gradient-synchronisation
hot path (bucket plan, flatten, ring all-reduce with averaging, unflatten,
standalone reduce-scatter / all-gather / broadcast, the logarithmic-latency
all-reduce schedules and their choice by size) for p simulated ranks in one
gfx950 GPU's HBM.

The compute lives in libddpsim.so (HIP kernels behind the C ABI declared in
include/ddpsim.h); `binding` marshals torch tensors to it. `workloads` holds
the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    ALGO, AVG, DTYPE_BF16, DTYPE_F32, EXPORTS, MAX_RANKS, SCHEDULES, CallTimer, CommStats,
    DDPError, Plan, Reducer,
    BROADCAST_BUCKET_BYTES, NOALLOC_SCRATCH_BYTES,
    allgather_sim, allreduce_sim, allreduce_sim_workspace, broadcast_coalesced, broadcast_sim,
    choose_schedule, ddp_allreduce_bucket, ddp_allreduce_buckets, ddp_broadcast_coalesced,
    ddp_bucket_plan, ddp_coalesce_plan, ddp_flatten, ddp_unflatten, sync_module_states,
    grad_pointer_table, load_library, overlap_step_time, reduce_scatter_sim, ring_allreduce_sim,
    ring_allreduce_sim_noalloc, ring_allreduce_sim_steps, ring_allreduce_sim_workspace,
    schedule_time,
)
