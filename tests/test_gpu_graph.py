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


@pytest.mark.parametrize("bf16", [False, True])
def test_graph_replay_of_step_by_step_schedules(oracle, bf16):
    """Every schedule step by step (one launch per message round, the bf16
    ones through their fp32 workspace) captured in one graph; each replay on
    fresh inputs, with eager work in between, gives the oracle's bits."""
    p, n = 5, 4099
    scheds = ("ring", "recursive_doubling", "rabenseifner", "tree")
    dt = torch.bfloat16 if bf16 else torch.float32
    code = 1 if bf16 else 0
    bufs = {s: [torch.empty(n, dtype=dt, device="cuda") for _ in range(p)] for s in scheds}
    ws = {}
    for s in scheds:
        need = ddp.allreduce_sim_workspace(p, n, code, s, True)
        ws[s] = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None

    def host_vals(seed):
        h = [W.normal_np(n, 1.0, seed, r) for r in range(p)]
        return [oracle.f32_to_bf16(x) for x in h] if bf16 else h

    def fill(vals):
        for s in scheds:
            for r in range(p):
                src = torch.from_numpy(vals[r].view("int16") if bf16 else vals[r])
                bufs[s][r].copy_(src.view(torch.bfloat16) if bf16 else src)

    def work():
        for s in scheds:
            ddp.allreduce_sim(bufs[s], s, True, avg="world", workspace=ws[s])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fill(host_vals(1))
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for seed in (11, 12, 11):
        vals = host_vals(seed)
        fill(vals)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in scheds:
            want, _ = oracle.allreduce(vals, s, avg="world", want_log=False)
            for r in range(p):
                assert_bits_equal(to_host(bufs[s][r]), want[r], f"seed {seed} {s} rank {r}")
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
