"""The library's launches inside a captured HIP graph: replaying the graph
several times, with fresh inputs and eager work in between, must give the
eager result bit for bit every time."""
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_host

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager(oracle):
    p = 4
    sizes = [3000, 17, 40_000, 5, 12_345]
    plan = ddp.ddp_bucket_plan(sizes, 4, 64 * 1024, 8 * 1024).upload().upload_segments(p)
    grads = [[torch.empty(n, device="cuda") for n in sizes] for _ in range(p)]
    table = ddp.grad_pointer_table(grads)
    tensors = [torch.empty(1001, device="cuda") for _ in range(p)]

    def fill(seed):
        for r in range(p):
            for i, n in enumerate(sizes):
                grads[r][i].copy_(torch.from_numpy(W.normal_np(n, 1.0, seed, r, stream=i)))
            tensors[r].copy_(torch.from_numpy(W.normal_np(1001, 1.0, seed + 7, r)))

    def work():
        for b in range(plan.num_buckets):
            ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
        ddp.ring_allreduce_sim(tensors, avg="world")

    # eager reference for each seed
    want = {}
    for seed in (1, 2, 3):
        fill(seed)
        work()
        torch.cuda.synchronize()
        want[seed] = ([[to_host(g) for g in rank] for rank in grads],
                      [to_host(t) for t in tensors])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fill(1)
        work()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for seed in (1, 2, 3, 2):
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager_g, eager_t = want[seed]
        for r in range(p):
            for i in range(len(sizes)):
                assert_bits_equal(to_host(grads[r][i]), eager_g[r][i], f"seed {seed} rank {r} param {i}")
            assert_bits_equal(to_host(tensors[r]), eager_t[r], f"seed {seed} tensor rank {r}")
        # eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
