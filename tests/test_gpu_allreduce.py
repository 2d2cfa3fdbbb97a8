"""GPU parity: ring all-reduce through the C ABI against the CPU oracle.

The bar: bit-exact in fp32 (same fold order, same correctly rounded division)
and in bf16 (fp32 fold, one round-to-nearest-even), for both algorithms
(fused single pass and the step-by-step ring), every averaging mode, ragged
sizes (padding, chunk boundaries inside a 16-byte vector, empty chunks,
several tiles per chunk) and p from 1 to 64.
"""
import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_dev, to_host, tokens_for

pytestmark = pytest.mark.gpu

CASES = [(1, 0), (1, 7), (2, 1), (2, 9), (3, 10), (4, 10), (4, 1_000_003), (5, 3),
         (5, 4099), (7, 50), (8, 8), (8, 61), (8, 8 * 65536 + 5), (13, 100_003),
         (16, 257), (33, 137), (40, 40_003), (48, 1_000), (64, 200), (64, 100_000)]


def _run(host, avg, tokens, algo):
    bufs = [to_dev(h) for h in host]
    ws = None
    p, n = len(host), host[0].size
    need = ddp.ring_allreduce_sim_workspace(p, n, 1 if host[0].dtype == np.uint16 else 0, algo)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=bufs[0].device)
    st = ddp.ring_allreduce_sim(bufs, avg=avg, tokens=tokens, algo=algo, workspace=ws)
    torch.cuda.synchronize()
    return [to_host(b) for b in bufs], st


@pytest.mark.parametrize("algo", ["fused", "ring"])
@pytest.mark.parametrize("avg", ["none", "world", "tokens"])
@pytest.mark.parametrize("p,n", CASES)
def test_allreduce_f32_bit_exact(oracle, p, n, avg, algo):
    host = [W.normal_np(n, 1.0, 100 + p, r) for r in range(p)]
    tokens = tokens_for(p) if avg == "tokens" else None
    got, st = _run(host, avg, tokens, algo)
    want, log = oracle.ring_allreduce(host, avg=avg, tokens=tokens)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"rank {r}")
    assert st.steps == 2 * (p - 1) and st.messages == len(log)
    if n:
        assert st.bytes_sent_per_rank == sum(m.bytes for m in log if m.src == 0)
        assert st.total_bytes == sum(m.bytes for m in log)


@pytest.mark.parametrize("algo", ["fused", "ring"])
@pytest.mark.parametrize("p,n", [(2, 1), (3, 10), (4, 1_000_003), (8, 4097), (8, 1 << 20),
                                 (16, 100_000), (33, 5_003), (64, 1_031), (64, 65_536 + 3)])
def test_allreduce_bf16_bit_exact(oracle, p, n, algo):
    host = [oracle.f32_to_bf16(W.normal_np(n, 1e-2, 200 + p, r)) for r in range(p)]
    got, _ = _run(host, "world", None, algo)
    want, _ = oracle.ring_allreduce(host, avg="world", want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"rank {r}")
    # the stated tolerance against an fp64 sum of the bf16 inputs
    x = np.stack([oracle.bf16_to_f32(h) for h in host]).astype(np.float64)
    s = x.sum(0) / p
    y = oracle.bf16_to_f32(got[0]).astype(np.float64)
    scale = np.abs(x).sum(0) / p
    assert np.all(np.abs(y - s) <= 1e-2 * np.abs(s) + (p - 1) * 2.0 ** -24 * scale + 1e-45)


@pytest.mark.parametrize("algo", ["fused", "ring"])
@pytest.mark.parametrize("p,n", [(3, 10), (4, 1003), (5, 23), (8, 61), (8, 4096 * 8 + 12), (64, 130)])
def test_order_probes(oracle, p, n, algo):
    """The oracle's order probes, run on the GPU. Probe A (1.0 on rank c,
    2^-24 on ranks c+1 and c+2, c the element's chunk) gives exactly 1.0 only
    when the fold starts at rank c rather than c+1; probe B (2^-24 on ranks c
    and c+1, 1.0 on rank c-1) gives 1 + 2^-23 only when it starts at rank c
    rather than c-1 or runs backwards."""
    C = -(-n // p)
    chunk = np.arange(n) // C
    host = [np.zeros(n, np.float32) for _ in range(p)]
    for i in range(n):
        c = int(chunk[i])
        host[c][i] = 1.0
        host[(c + 1) % p][i] += np.float32(2.0 ** -24)
        host[(c + 2) % p][i] += np.float32(2.0 ** -24)
    got, _ = _run(host, "none", None, algo)
    assert np.all(got[0] == np.float32(1.0))
    host_b = [np.zeros(n, np.float32) for _ in range(p)]
    for i in range(n):
        c = int(chunk[i])
        host_b[c][i] = np.float32(2.0 ** -24)
        host_b[(c + 1) % p][i] += np.float32(2.0 ** -24)
        host_b[(c - 1) % p][i] += np.float32(1.0)
    got, _ = _run(host_b, "none", None, algo)
    assert np.all(got[0] == np.float32(1.0 + 2.0 ** -23))


@pytest.mark.parametrize("p,n", [(2, 7), (3, 1000), (4, 1_000_003), (8, 100_001)])
def test_ring_intermediate_states(oracle, p, n):
    host = [W.normal_np(n, 1.0, 300 + p, r) for r in range(p)]
    bufs = [to_dev(h) for h in host]
    for s in range(2 * (p - 1)):
        ddp.ring_allreduce_sim_steps(bufs, s, 1, avg="world")
        torch.cuda.synchronize()
        want, _ = oracle.ring_allreduce(host, avg="world", max_steps=s + 1, want_log=False)
        for r in range(p):
            assert_bits_equal(to_host(bufs[r]), want[r], f"step {s} rank {r}")


def test_integer_inputs_exact(oracle):
    p, n = 16, 300_007
    host = [W.integer_valued_np(n, 9, r) for r in range(p)]
    got, _ = _run(host, "none", None, "fused")
    total = np.sum(np.stack(host).astype(np.int64), axis=0)
    assert np.array_equal(got[5].astype(np.int64), total)


def test_subnormals_and_signed_zeros(oracle):
    p, n = 4, 4099
    rng = np.random.default_rng(5)
    host = []
    for r in range(p):
        bitsv = rng.integers(0, 1 << 23, size=n).astype(np.uint32)  # subnormal mantissas
        bitsv |= (rng.integers(0, 2, size=n).astype(np.uint32) << 31)
        h = bitsv.view(np.float32).copy()
        h[::7] = -0.0
        host.append(h)
    host[0][::13] = 0.0
    for avg in ("none", "world", "tokens"):
        tokens = [3, 5, 7, 11] if avg == "tokens" else None
        got, _ = _run(host, avg, tokens, "fused")
        want, _ = oracle.ring_allreduce(host, avg=avg, tokens=tokens, want_log=False)
        for r in range(p):
            assert_bits_equal(got[r], want[r], f"{avg} rank {r}")


def test_buffers_are_independent_allocations_at_offsets(oracle):
    """Rank buffers carved from one allocation at 16-byte aligned offsets."""
    p, n = 5, 12_345
    host = [W.normal_np(n, 1.0, 77, r) for r in range(p)]
    stride = (n + 3) // 4 * 4 + 4
    big = torch.zeros(p * stride + 8, dtype=torch.float32, device="cuda")
    bufs = [big[r * stride + 4: r * stride + 4 + n] for r in range(p)]
    for b, h in zip(bufs, host):
        b.copy_(torch.from_numpy(h))
    ddp.ring_allreduce_sim(bufs, avg="world")
    torch.cuda.synchronize()
    want, _ = oracle.ring_allreduce(host, avg="world", want_log=False)
    for r in range(p):
        assert_bits_equal(to_host(bufs[r]), want[r])
    # guard elements between ranks untouched
    g = big.cpu().numpy()
    for r in range(p):
        assert np.all(g[r * stride: r * stride + 4] == 0)


@pytest.mark.parametrize("bf16,p,n", [(True, 8, 17_000_003), (False, 13, 6_000_001),
                                       (True, 20, 7_000_003), (False, 29, 2_400_001),
                                       (True, 64, 2_200_001), (False, 64, 1_100_000)])
def test_fused_past_the_infinity_cache(oracle, bf16, p, n):
    """Rank buffers totalling more than 256 MiB take the fused kernel's
    streaming shape (non-temporal accesses; beyond 8 ranks the ranks of a
    tile are split over 2 or 8 waves whose running sum passes through LDS):
    every element against the oracle, with a divisor that is not a power of
    two."""
    host = [W.normal_np(n, 1.0, 900 + p, r) for r in range(p)]
    if bf16:
        host = [oracle.f32_to_bf16(h) for h in host]
    assert p * n * (2 if bf16 else 4) > 256 << 20
    tokens = tokens_for(p, 5)
    got, _ = _run(host, "tokens", tokens, "fused")
    want, _ = oracle.ring_allreduce(host, avg="tokens", tokens=tokens, want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"rank {r}")


# Sizes on both sides of each rule that picks the fused kernel's form: the
# small-call bound (at most 256 workgroups of 256 threads x 2 vectors), which
# takes the 8-wave form beyond 32 ranks and the 32-load one-vector form at
# 9-32 ranks, and the 256 MiB streaming bound, past which 8 ranks keep one
# wave per tile, 9-27 ranks take 2 waves and 28 or more take 8.
FORM_EDGES = [
    (False, 64, 524_288), (False, 64, 524_289),      # 256 | 320 workgroups
    (False, 33, 473_088), (False, 33, 473_089),      # 231 | 264
    (False, 32, 524_288), (False, 32, 524_289),      # 256 | 288
    (True, 64, 1_048_576), (True, 64, 1_048_577),    # bf16: 256 | 320
    (False, 8, 8_388_609),                           # streaming, one wave
    (False, 9, 7_456_541),                           # streaming, 2 waves
    (False, 27, 2_485_513), (False, 27, 2_485_514),  # cached | streaming, 2 waves
    (False, 28, 2_396_746),                          # streaming, 8 waves
]


@pytest.mark.parametrize("bf16,p,n", FORM_EDGES)
def test_fused_launch_form_edges(oracle, bf16, p, n):
    """Every element against the oracle on either side of each launch-form
    rule of the fused all-reduce, token-weighted (a divisor that is not a
    power of two)."""
    eb = 2 if bf16 else 4
    if p == 27:
        assert (p * n * eb > 256 << 20) == (n % 2 == 0)
    host = [W.normal_np(n, 1.0, 970 + p, r) for r in range(p)]
    if bf16:
        host = [oracle.f32_to_bf16(h) for h in host]
    tokens = tokens_for(p, 7)
    got, _ = _run(host, "tokens", tokens, "fused")
    want, _ = oracle.ring_allreduce(host, avg="tokens", tokens=tokens, want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"rank {r}")


def test_ring_steps_past_the_infinity_cache(oracle):
    """Rank buffers totalling more than 256 MiB take the ring step's
    streaming shape (one-wave workgroups, non-temporal accesses): every
    intermediate state of a ragged n against the oracle's, every element,
    with a divisor that is not a power of two."""
    p, n = 5, 14_000_003
    assert p * n * 4 > 256 << 20
    host = [W.normal_np(n, 1.0, 950, r) for r in range(p)]
    bufs = [to_dev(h) for h in host]
    tokens = tokens_for(p, 6)
    for s in range(2 * (p - 1)):
        ddp.ring_allreduce_sim_steps(bufs, s, 1, avg="tokens", tokens=tokens)
        torch.cuda.synchronize()
        want, _ = oracle.ring_allreduce(host, avg="tokens", tokens=tokens, max_steps=s + 1,
                                        want_log=False)
        for r in range(p):
            assert_bits_equal(to_host(bufs[r]), want[r], f"step {s} rank {r}")


def test_bf16_ring_past_the_infinity_cache(oracle):
    """The bf16 ring's fp32 workspace rows past 256 MiB: the whole call."""
    p, n = 8, 9_000_001
    host = [oracle.f32_to_bf16(W.normal_np(n, 1.0, 960, r)) for r in range(p)]
    assert p * n * 4 > 256 << 20
    got, _ = _run(host, "world", None, "ring")
    want, _ = oracle.ring_allreduce(host, avg="world", want_log=False)
    for r in range(p):
        assert_bits_equal(got[r], want[r], f"rank {r}")
