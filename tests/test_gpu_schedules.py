"""GPU parity: all-reduce under the logarithmic-latency schedules (recursive
doubling, Rabenseifner, tree) through the C ABI against the CPU oracle's
literal simulations.

The bar: bit-exact in fp32 and bf16 for both forms (one fused pass, and the
schedule step by step), every averaging mode, p from 1 to 64 (powers of two
and not), ragged sizes (tails shorter than a vector, Rabenseifner chunks that
straddle vectors or lie wholly in the padding, several tiles per job), the
cancellation probes that pin each schedule's pairing, and the accounting
against the oracle's message log. At a size the oracle does not simulate
whole (64 ranks of 16 MiB), sampled elements are checked against the
oracle's per-element form; the crossover sweep's largest case (4 ranks of
64 MB) is compared whole.
"""
import itertools

import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_dev, to_host, tokens_for

pytestmark = pytest.mark.gpu

LOG_SCHEDULES = ("recursive_doubling", "rabenseifner", "tree")
CASES = [(1, 0), (1, 9), (2, 1), (2, 4099), (3, 10), (4, 1003), (5, 3), (5, 4099),
         (6, 77), (7, 50), (8, 8), (8, 61), (8, 8 * 4096 + 5), (9, 1000), (13, 100_003),
         (16, 257), (31, 600), (32, 33), (33, 1000), (63, 129), (64, 200), (64, 70_001)]


def _run(host, schedule, steps, avg="none", tokens=None):
    bufs = [to_dev(h) for h in host]
    p, n = len(host), host[0].size
    code = 1 if host[0].dtype == np.uint16 else 0
    need = ddp.allreduce_sim_workspace(p, n, code, schedule, steps)
    ws = torch.empty(need, dtype=torch.uint8, device=bufs[0].device) if need else None
    st = ddp.allreduce_sim(bufs, schedule, steps, avg=avg, tokens=tokens, workspace=ws)
    torch.cuda.synchronize()
    return [to_host(b) for b in bufs], st


@pytest.mark.parametrize("steps", [False, True])
@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
@pytest.mark.parametrize("avg", ["none", "world", "tokens"])
@pytest.mark.parametrize("p,n", CASES)
def test_f32_bit_exact(oracle, p, n, avg, schedule, steps):
    host = [W.normal_np(n, 1.0, 300 + p, r) for r in range(p)]
    tokens = tokens_for(p) if avg == "tokens" else None
    got, st = _run(host, schedule, steps, avg, tokens)
    want, log = oracle.allreduce(host, schedule, avg=avg, tokens=tokens)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"{schedule} steps={steps} rank {r}")
    assert st.messages == len(log)
    assert st.steps == len({(m.phase, m.step) for m in log})
    assert st.total_bytes == sum(m.bytes for m in log)
    if log:
        assert st.bytes_sent_per_rank == max(
            sum(m.bytes for m in log if m.src == r) for r in range(p))
        assert st.bytes_recv_per_rank == max(
            sum(m.bytes for m in log if m.dst == r) for r in range(p))


@pytest.mark.parametrize("steps", [False, True])
@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
@pytest.mark.parametrize("p,n", [(2, 1), (3, 10), (4, 1_000_003), (5, 4097), (8, 1 << 20),
                                 (12, 100_000), (64, 65_536 + 3)])
def test_bf16_bit_exact(oracle, p, n, schedule, steps):
    host = [oracle.f32_to_bf16(W.normal_np(n, 1e-2, 400 + p, r)) for r in range(p)]
    got, _ = _run(host, schedule, steps, "world")
    want, _ = oracle.allreduce(host, schedule, avg="world", want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"{schedule} steps={steps} rank {r}")
    # the stated tolerance against an fp64 sum of the bf16 inputs
    x = np.stack([oracle.bf16_to_f32(h) for h in host]).astype(np.float64)
    s = x.sum(0) / p
    y = oracle.bf16_to_f32(got[0]).astype(np.float64)
    scale = np.abs(x).sum(0) / p
    assert np.all(np.abs(y - s) <= 1e-2 * np.abs(s) + (p - 1) * 2.0 ** -24 * scale + 1e-45)


@pytest.mark.parametrize("steps", [False, True])
@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
@pytest.mark.parametrize("p", [3, 5, 8, 12, 16])
def test_cancellation_probes(oracle, schedule, p, steps):
    """+1 at rank a, -1 at rank b, 2^-30 at rank c, one element per ordered
    triple: the result is 2^-30 exactly when a and b are summed before c
    joins them, which the schedule's pairing decides."""
    triples = list(itertools.permutations(range(p), 3))
    n = len(triples)
    host = [np.zeros(n, np.float32) for _ in range(p)]
    for i, (a, b, c) in enumerate(triples):
        host[a][i], host[b][i], host[c][i] = 1.0, -1.0, 2.0 ** -30
    got, _ = _run(host, schedule, steps)
    want, _ = oracle.allreduce(host, schedule, want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"rank {r}")


@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
def test_fused_and_steps_agree_with_ring_on_integers(oracle, schedule):
    """Integer-valued inputs sum exactly in any order, so every schedule and
    the ring give the same bits."""
    p, n = 11, 50_001
    host = [W.integer_valued_np(n, 3, r) for r in range(p)]
    a, _ = _run(host, schedule, False)
    b, _ = _run(host, schedule, True)
    c, _ = _run(host, "ring", False)
    for r in range(p):
        assert_bits_equal(a[r], c[r]) and assert_bits_equal(b[r], c[r])


@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
def test_full_size_sampled(oracle, schedule):
    """64 ranks of 4 Mi fp32 elements (16 MiB each, the non-temporal path),
    token-averaged; 4096 sampled elements against the per-element form."""
    p, n = 64, (1 << 22) + 5
    dev = torch.device("cuda", 0)
    bufs = [W.normal_torch(n, 1.0, 77, r, dev) for r in range(p)]
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([rng.integers(0, n, 4096), [0, n - 1, n - 5]]))
    ti = torch.from_numpy(idx).to(dev)
    vals = np.stack([b[ti].cpu().numpy() for b in bufs], axis=1)
    tokens = tokens_for(p, 3)
    ddp.allreduce_sim(bufs, schedule, False, avg="tokens", tokens=tokens)
    torch.cuda.synchronize()
    want = oracle.tree_allreduce_at(vals, schedule, avg="tokens", tokens=tokens)
    for r in (0, 17, 63):
        assert_bits_equal(bufs[r][ti].cpu().numpy(), want, f"rank {r}")


def test_ring_schedule_is_ring_allreduce_sim(oracle):
    p, n = 7, 10_007
    host = [W.normal_np(n, 1.0, 9, r) for r in range(p)]
    for steps in (False, True):
        got, st = _run(host, "ring", steps, "world")
        want, log = oracle.ring_allreduce(host, avg="world")
        for r in range(p):
            assert_bits_equal(got[r], want[r])
        assert st.steps == 2 * (p - 1) and st.messages == len(log)


def test_fused_hbm_bytes_and_step_traffic():
    p, n = 8, 4096
    host = [W.normal_np(n, 1.0, 1, r) for r in range(p)]
    _, fused = _run(host, "recursive_doubling", False)
    assert fused.hbm_bytes == 2 * p * n * 4
    _, stepped = _run(host, "recursive_doubling", True)
    assert stepped.hbm_bytes == 3 * (p // 2) * 4 * n * 4  # 3 steps, p/2 pairs, 2 reads + 2 writes


@pytest.mark.parametrize("schedule", ("ring",) + LOG_SCHEDULES)
def test_crossover_sweep_largest_size_whole(oracle, schedule):
    """The crossover sweep's largest case, 4 ranks of 64 MB averaged by p,
    in both forms the sweep times (step by step and fused): every element
    against the oracle's literal simulation."""
    p, n = 4, 1 << 24
    host = [W.normal_np(n, 1.0, 700, r) for r in range(p)]
    want, _ = oracle.allreduce(host, schedule, avg="world", want_log=False)
    for steps in (True, False):
        got, _ = _run(host, schedule, steps, "world")
        for r in range(p):
            assert_bits_equal(got[r], want[r], f"{schedule} steps={steps} rank {r}")


@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
@pytest.mark.parametrize("p,n,bf16,avg", [
    (16, 4_194_305, False, "world"),   # a tail shorter than a vector
    (24, 5_592_408, True, "tokens"),
    (40, 1_677_723, False, "none"),
    (64, 1_048_579, False, "tokens"),
])
def test_fused_many_ranks_past_the_infinity_cache(oracle, schedule, p, n, bf16, avg):
    """From 16 ranks of buffers past the Infinity Cache the fused kernel
    gives each wave of a workgroup one batch of eight leaves and joins the
    batch sums through LDS: every element of every rank against the
    oracle's literal schedule."""
    assert p * n * (2 if bf16 else 4) > 256 << 20
    host = [W.normal_np(n, 1.0, 800 + p, r) for r in range(p)]
    if bf16:
        host = [oracle.f32_to_bf16(h) for h in host]
    tokens = tokens_for(p, 4) if avg == "tokens" else None
    got, _ = _run(host, schedule, False, avg, tokens)
    want, _ = oracle.allreduce(host, schedule, avg=avg, tokens=tokens, want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"{schedule} rank {r}")


# Sizes on both sides of each rule that picks the fused schedules' form from
# 16 ranks: at most 512 one-wave tiles, or buffers past 256 MiB, take one
# batch of eight leaves per wave; 16 ranks of exactly 256 MiB, and 15 ranks
# past it (eight core ranks), keep one wave per tile.
@pytest.mark.parametrize("schedule", LOG_SCHEDULES)
@pytest.mark.parametrize("p,n", [
    (16, 131_071), (16, 131_072),    # 512 tiles | 513
    (64, 131_071), (64, 131_072),
    (16, 4_194_304),                 # 256 MiB exactly: one wave
    (15, 4_473_925),                 # past 256 MiB, Q = 8: one wave
])
def test_fused_launch_form_edges(oracle, schedule, p, n):
    """Every element of every rank against the oracle's literal schedule,
    token-weighted."""
    host = [W.normal_np(n, 1.0, 820 + p, r) for r in range(p)]
    tokens = tokens_for(p, 9)
    got, _ = _run(host, schedule, False, "tokens", tokens)
    want, _ = oracle.allreduce(host, schedule, avg="tokens", tokens=tokens, want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"{schedule} rank {r}")
