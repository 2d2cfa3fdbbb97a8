"""GPU parity for the coalesced broadcast (init-time synchronisation of
parameters and buffers, and the per-forward buffer broadcast) and for the
bucket rebuild from the observed ready order, through the C ABI against the
CPU oracle.

The bar: every rank's copy of every tensor holds the root's bytes exactly,
bytes outside the tensors are untouched, the stats equal the oracle's
message log; after a rebuild the bucket all-reduce over the rebuilt plan is
bit-exact against the oracle's flatten -> ring -> unflatten over the plan
the oracle builds from the same order.
"""
import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, make_grads, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 7, 4095, 4096, 4097, 12_345, 65_536 + 3, 100_000, 2]
NP_OF = {torch.float32: np.float32, torch.bfloat16: np.uint16, torch.int64: np.int64,
         torch.uint8: np.uint8}


def _arena_views(p, sizes, dtype, layout, seed):
    """Rank r's tensors as views into one arena of seeded values (the bytes
    between and after the views must survive the broadcast). "aligned":
    every view starts on a 16-element boundary; "odd": the same odd offsets
    on every rank; "mixed": each rank shifted differently."""
    rng = np.random.default_rng(seed)
    arenas, views, hosts = [], [], []
    for r in range(p):
        gap = {"aligned": 0, "odd": 1, "mixed": r % 3 + 1}[layout]
        offs, off = [], gap
        for n in sizes:
            offs.append(off)
            off += n + 16 + gap
            if layout == "aligned":
                off = (off + 15) // 16 * 16
        total = off + 16
        if dtype in (torch.float32, torch.bfloat16):
            a = torch.from_numpy(W.normal_np(total, 1.0, seed, r)).to("cuda").to(dtype)
        else:
            hi = 250 if dtype == torch.uint8 else 1 << 40
            a = torch.from_numpy(rng.integers(0, hi, size=total).astype(NP_OF[dtype])).to("cuda")
        arenas.append(a)
        views.append([a[o:o + n] for o, n in zip(offs, sizes)])
        hosts.append(to_host(a))
    return arenas, views, hosts


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int64, torch.uint8])
@pytest.mark.parametrize("layout", ["aligned", "odd", "mixed"])
@pytest.mark.parametrize("p,root", [(1, 0), (2, 1), (3, 0), (5, 4), (8, 5), (13, 7), (17, 16),
                                    (64, 63)])
def test_broadcast_coalesced_bit_exact(oracle, dtype, layout, p, root):
    arenas, views, before = _arena_views(p, SIZES, dtype, layout, 31 * p + root)
    eb = torch.tensor([], dtype=dtype).element_size()
    cap = 20_000 * eb  # several buckets
    host_t = [[to_host(v) for v in views[r]] for r in range(p)]
    plan = ddp.ddp_coalesce_plan(SIZES, eb, cap).upload()
    table = ddp.grad_pointer_table(views)
    st = ddp.ddp_broadcast_coalesced(plan, table, p, root)
    torch.cuda.synchronize()
    want, log, bof = oracle.broadcast_coalesced(host_t, root=root, cap_bytes=cap)
    assert plan.buckets() == oracle.coalesce_plan(SIZES, eb, cap).buckets()
    for r in range(p):
        for i, v in enumerate(views[r]):
            got = to_host(v)
            assert np.array_equal(got.view(np.uint8), want[r][i].view(np.uint8)), (r, i)
        # bytes outside the tensors are untouched
        after = to_host(arenas[r])
        mask = np.ones(after.size, bool)
        for v in views[r]:
            o = v.storage_offset()
            mask[o:o + v.numel()] = False
        assert np.array_equal(after[mask].view(np.uint8), before[r][mask].view(np.uint8))
    assert st.messages == len(log)
    assert st.steps == len({m.step for m in log})
    assert st.total_bytes == sum(m.bytes for m in log)
    if log:
        assert st.bytes_sent_per_rank == max(sum(m.bytes for m in log if m.src == r)
                                             for r in range(p))
        assert st.bytes_recv_per_rank == max(sum(m.bytes for m in log if m.dst == r)
                                             for r in range(p))
    assert st.hbm_bytes == p * sum(SIZES) * eb


def test_sync_module_states_makes_replicas_identical(oracle):
    """Parameters (fp32) and buffers (fp32 running statistics and an int64
    step counter) of 8 ranks become rank 0's: one coalesced broadcast per
    element size, the default 250 MiB cap."""
    p = 8
    shapes = [W.numel(s) for _, s in W.gpt2_small_params()[:14]]
    params = [[to_dev(W.normal_np(n, 1e-2, 9, r, stream=i)) for i, n in enumerate(shapes)]
              for r in range(p)]
    buffers = [[to_dev(W.normal_np(768, 1.0, 10, r)), to_dev(W.normal_np(768, 1.0, 11, r)),
                torch.tensor([100 + r], dtype=torch.int64, device="cuda")] for r in range(p)]
    want_p = [to_host(t) for t in params[0]]
    want_b = [to_host(t) for t in buffers[0]]
    stats = ddp.sync_module_states(params, buffers, root=0)
    torch.cuda.synchronize()
    assert len(stats) == 2  # 4-byte and 8-byte groups
    for r in range(p):
        for t, w in zip(params[r], want_p):
            assert_bits_equal(to_host(t), w)
        for t, w in zip(buffers[r], want_b):
            assert np.array_equal(to_host(t), w)


def test_buffer_broadcast_from_authoritative_rank_on_a_side_stream(oracle):
    """The per-forward buffer broadcast from a non-zero authoritative rank,
    issued on another stream: the tables allocated on the current stream
    stay valid until the kernels there have run."""
    p = 4
    bufs = [[to_dev(W.normal_np(n, 1.0, 12, r)) for n in (3, 4096, 777)] for r in range(p)]
    want = [to_host(t) for t in bufs[2]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ddp.broadcast_coalesced(bufs, root=2, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(p):
        for t, w in zip(bufs[r], want):
            assert_bits_equal(to_host(t), w)


SIZES_R = [5000, 0, 7, 4096, 4097, 1, 33_333, 12, 0, 65_536 + 9, 3, 100_000]


@pytest.mark.parametrize("bf16", [False, True])
def test_rebuild_from_observed_ready_order(oracle, bf16):
    """First pass: gradients marked in a random order; the reducer reports
    that order. The buckets rebuilt from it (ddp_bucket_plan with order) are
    the oracle's, and a second pass over the rebuilt plan gives the oracle's
    flatten -> ring -> unflatten bits."""
    p = 4
    eb = 2 if bf16 else 4
    cap, first = 96 * 1024, 8 * 1024
    plan = ddp.ddp_bucket_plan(SIZES_R, eb, cap, first).upload_segments(p)
    host, grads = make_grads(p, SIZES_R, 1300, bf16, oracle, "mixed")
    table = ddp.grad_pointer_table(grads)
    order = [int(i) for i in np.random.default_rng(3).permutation(len(SIZES_R))]
    red = ddp.Reducer(plan, p, table, avg="world")
    red.prepare()
    for i in order:
        red.mark_ready(i)
    red.finalize()
    assert red.ready_order() == order
    torch.cuda.synchronize()
    # the first pass reduced the gradients once; restore them before the
    # pass over the rebuilt plan
    for r in range(p):
        for i in range(len(SIZES_R)):
            grads[r][i].copy_(to_dev(host[r][i]))
    rebuilt = ddp.ddp_bucket_plan(SIZES_R, eb, cap, first, order=red.ready_order())
    rebuilt.upload_segments(p)
    oplan = oracle.bucket_plan(SIZES_R, eb, cap, first, order=order)
    assert rebuilt.buckets() == oplan.buckets()
    red2 = ddp.Reducer(rebuilt, p, table, avg="world")
    red2.prepare()
    for i in order:
        red2.mark_ready(i)
    red2.finalize()
    torch.cuda.synchronize()
    # in the rebuilt plan the marks complete buckets in index order, so every
    # bucket is launched by the mark of its last parameter
    runs, total = oracle.reducer_schedule(oplan, order)
    assert red2.launch_log() == runs and total == rebuilt.num_buckets
    assert all(n == 1 for _, _, n in runs)
    want = [[g.copy() for g in rank] for rank in host]
    for b in range(oplan.num_buckets):
        flats = [oracle.flatten(want[r], oplan, b) for r in range(p)]
        red_, _ = oracle.ring_allreduce(flats, avg="world", want_log=False)
        for r in range(p):
            oracle.unflatten(red_[r], oplan, b, want[r])
    for r in range(p):
        for i in range(len(SIZES_R)):
            assert_bits_equal(to_host(grads[r][i]), want[r][i], f"rank {r} param {i}")


def test_gpt2_small_parameter_sync_full_size():
    """The benchmark's sync workload at its size: the 148 GPT-2-small fp32
    parameter tensors of 8 ranks (views into one arena per rank, 64-element
    aligned), two 250 MiB buckets, from rank 0. Every element of every rank
    must equal rank 0's."""
    p = 8
    sizes = [W.numel(s) for _, s in W.gpt2_small_params()]
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + 63) // 64 * 64
    arenas = [W.normal_torch(off, 1e-3, 2, r, torch.device("cuda", 0)) for r in range(p)]
    views = [[a[o:o + n] for o, n in zip(offs, sizes)] for a in arenas]
    want = torch.cat([v for v in views[0]]).clone()
    plan = ddp.ddp_coalesce_plan(sizes, 4, ddp.BROADCAST_BUCKET_BYTES).upload()
    assert plan.num_buckets == 2
    table = ddp.grad_pointer_table(views)
    st = ddp.ddp_broadcast_coalesced(plan, table, p, 0)
    torch.cuda.synchronize()
    assert st.messages == 2 * (p - 1) and st.hbm_bytes == p * sum(sizes) * 4
    for r in range(1, p):
        got = torch.cat([v for v in views[r]])
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), r
