"""GPU parity: standalone reduce-scatter, all-gather and broadcast against
the CPU oracle (bit-exact), in and out of place, with shards that are and
are not whole 16-byte vectors."""
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_dev, to_host, tokens_for

pytestmark = pytest.mark.gpu


def _vals(p, n, seed, bf16, oracle):
    h = [W.normal_np(n, 1.0, seed, r) for r in range(p)]
    return [oracle.f32_to_bf16(x) for x in h] if bf16 else h


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("avg", ["none", "world", "tokens"])
@pytest.mark.parametrize("p,C", [(1, 5), (2, 3), (3, 1001), (4, 4096), (8, 12_345), (8, 65_536),
                                 (16, 4099), (17, 4096), (64, 8), (64, 513)])
def test_reduce_scatter(oracle, p, C, avg, in_place, bf16):
    n = p * C
    host = _vals(p, n, 400 + p, bf16, oracle)
    tokens = tokens_for(p, 1) if avg == "tokens" else None
    ins = [to_dev(h) for h in host]
    if in_place:
        outs = [ins[r][r * C:(r + 1) * C] for r in range(p)]
    else:
        outs = [torch.empty(C, dtype=ins[0].dtype, device="cuda") for _ in range(p)]
    st = ddp.reduce_scatter_sim(ins, outs, avg=avg, tokens=tokens)
    torch.cuda.synchronize()
    want, log = oracle.reduce_scatter(host, avg=avg, tokens=tokens)
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), want[r], f"rank {r}")
    assert st.messages == len(log) and st.steps == p - 1
    assert st.bytes_sent_per_rank == sum(m.bytes for m in log if m.src == 0)


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("p,C", [(1, 7), (2, 3), (3, 1001), (4, 4096), (5, 333), (8, 12_345),
                                 (13, 777), (16, 100), (17, 55), (64, 9), (64, 1024)])
def test_allgather(oracle, p, C, bf16, in_place):
    host = _vals(p, C, 500 + p, bf16, oracle)
    dt = torch.bfloat16 if bf16 else torch.float32
    outs = [torch.full((p * C,), 7.0, dtype=dt, device="cuda") for _ in range(p)]
    if in_place:
        ins = [outs[r][r * C:(r + 1) * C] for r in range(p)]
        for r in range(p):
            ins[r].copy_(to_dev(host[r]))
    else:
        ins = [to_dev(h) for h in host]
    st = ddp.allgather_sim(ins, outs)
    torch.cuda.synchronize()
    want, log = oracle.allgather(host)
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), want[r], f"rank {r}")
    assert st.messages == len(log)
    assert st.bytes_sent_per_rank == sum(m.bytes for m in log if m.src == 0)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("p,n,src", [(1, 5, 0), (2, 1, 1), (5, 4099, 3), (8, 1 << 20, 0), (13, 1001, 12), (64, 70_001, 17)])
def test_broadcast(oracle, p, n, src, bf16):
    host = _vals(p, n, 600 + p, bf16, oracle)
    bufs = [to_dev(h) for h in host]
    st = ddp.broadcast_sim(bufs, src=src)
    torch.cuda.synchronize()
    want, log = oracle.broadcast(host, src)
    for r in range(p):
        assert_bits_equal(to_host(bufs[r]), want[r], f"rank {r}")
    assert st.messages == len(log) and st.steps == len({m.step for m in log})


def test_rs_then_ag_equals_allreduce_on_integers(oracle):
    p, C = 8, 10_001
    n = p * C
    host = [W.integer_valued_np(n, 3, r) for r in range(p)]
    ins = [to_dev(h) for h in host]
    outs = [torch.empty(n, device="cuda") for _ in range(p)]
    shards = [ins[r][r * C:(r + 1) * C] for r in range(p)]
    ddp.reduce_scatter_sim(ins, shards)
    ddp.allgather_sim(shards, outs)
    ar = [to_dev(h) for h in host]
    ddp.ring_allreduce_sim(ar)
    torch.cuda.synchronize()
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), to_host(ar[r]))


@pytest.mark.parametrize("op", ["broadcast", "allgather_in_place"])
def test_two_rank_copies_past_the_infinity_cache(oracle, op):
    """Two ranks of 150 Mi elements (600 MB each): the copy whose every
    source byte goes to one destination, which streams both its loads and its
    stores, against the oracle (the broadcast with a tail of 8 bytes past the
    last 16-byte vector; the all-gather's shards whole vectors)."""
    p, n = 2, 150 * (1 << 20) + (6 if op == "broadcast" else 8)
    host = _vals(p, n, 650, False, oracle)
    if op == "broadcast":
        bufs = [to_dev(h) for h in host]
        ddp.broadcast_sim(bufs, src=1)
        torch.cuda.synchronize()
        want, _ = oracle.broadcast(host, 1)
    else:
        C = n // p
        shards = [h[r * C:(r + 1) * C] for r, h in enumerate(host)]
        bufs = [to_dev(h) for h in host]
        ddp.allgather_sim([bufs[r][r * C:(r + 1) * C] for r in range(p)], bufs)
        torch.cuda.synchronize()
        want, _ = oracle.allgather(shards)
    for r in range(p):
        assert_bits_equal(to_host(bufs[r]), want[r], f"rank {r}")


@pytest.mark.parametrize("p", [2, 3, 5])
def test_few_ranks_past_the_infinity_cache(oracle, p):
    """Fewer than 8 ranks of large buffers: the fused all-reduce and the
    reduce-scatter take a residency bound scaled by the rank count; every
    element against the oracle."""
    C = (300 << 20) // (4 * p) // 4 * 4 + 4
    n = p * C
    host = _vals(p, n, 660 + p, False, oracle)
    tokens = tokens_for(p, 2)
    ins = [to_dev(h) for h in host]
    outs = [torch.empty(C, device="cuda") for _ in range(p)]
    ddp.reduce_scatter_sim(ins, outs, avg="tokens", tokens=tokens)
    ddp.ring_allreduce_sim(ins, avg="tokens", tokens=tokens)
    torch.cuda.synchronize()
    want, _ = oracle.reduce_scatter(host, avg="tokens", tokens=tokens)
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), want[r], f"reduce-scatter rank {r}")
    want, _ = oracle.ring_allreduce(host, avg="tokens", tokens=tokens, want_log=False)
    for r in range(p):
        assert_bits_equal(to_host(ins[r]), want[r], f"all-reduce rank {r}")


@pytest.mark.parametrize("p,C,bf16,in_place,avg", [
    (17, 240_004, False, False, "world"),   # chunks off the 64-vector tile grid
    (20, 336_008, True, True, "tokens"),
    (40, 83_896, True, False, "none"),
    (64, 16_388, False, True, "tokens"),
    (64, 16_390, False, False, "world"),    # shards not whole vectors: element path
])
def test_reduce_scatter_many_ranks_past_the_infinity_cache(oracle, p, C, bf16, in_place, avg):
    """Beyond 16 ranks of inputs past the Infinity Cache the reduce-scatter
    splits a tile's ranks over two waves whose running sum passes through
    LDS: every element of every shard against the oracle."""
    n = p * C
    assert p * n * (2 if bf16 else 4) > 256 << 20
    host = _vals(p, n, 670 + p, bf16, oracle)
    tokens = tokens_for(p, 3) if avg == "tokens" else None
    ins = [to_dev(h) for h in host]
    if in_place:
        outs = [ins[r][r * C:(r + 1) * C] for r in range(p)]
    else:
        outs = [torch.empty(C, dtype=ins[0].dtype, device="cuda") for _ in range(p)]
    ddp.reduce_scatter_sim(ins, outs, avg=avg, tokens=tokens)
    torch.cuda.synchronize()
    want, _ = oracle.reduce_scatter(host, avg=avg, tokens=tokens)
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), want[r], f"rank {r}")


# Shard sizes on both sides of each rule that picks the reduce-scatter's
# form beyond 16 ranks (whole-vector shards): at most 512 tiles of 64 vectors
# take 8 waves per tile, inputs past 256 MiB take 2, the rest 256 threads x
# 2 vectors; 16 ranks keep one wave per tile.
@pytest.mark.parametrize("p,C", [
    (17, 7_680), (17, 7_684),        # 510 tiles | 544
    (64, 2_048), (64, 2_052),        # 512 | 640
    (17, 232_208), (17, 232_212),    # cached | past 256 MiB
    (16, 7_680),                     # 480 tiles, one wave
])
def test_reduce_scatter_launch_form_edges(oracle, p, C):
    """Every element of every shard against the oracle, token-weighted, in
    place for even C / 4 and out of place otherwise."""
    n = p * C
    if (p, C) in ((17, 232_208), (17, 232_212)):
        assert (p * n * 4 > 256 << 20) == (C == 232_212)
    in_place = (C // 4) % 2 == 0
    host = _vals(p, n, 690 + p, False, oracle)
    tokens = tokens_for(p, 8)
    ins = [to_dev(h) for h in host]
    if in_place:
        outs = [ins[r][r * C:(r + 1) * C] for r in range(p)]
    else:
        outs = [torch.empty(C, dtype=ins[0].dtype, device="cuda") for _ in range(p)]
    ddp.reduce_scatter_sim(ins, outs, avg="tokens", tokens=tokens)
    torch.cuda.synchronize()
    want, _ = oracle.reduce_scatter(host, avg="tokens", tokens=tokens)
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), want[r], f"rank {r}")


# The fan-out copy splits a tile's destinations over W waves, W the smallest
# power of two with 4 W >= destinations (at most 8): rank counts on both
# sides of each step, and the 256 MiB bound past which its stores stream.
@pytest.mark.parametrize("p,n,src", [
    (5, 100_003, 4), (6, 100_003, 0),    # 4 destinations: 1 wave | 5: 2 waves
    (9, 100_003, 8), (10, 100_003, 3),   # 8: 2 | 9: 4
    (17, 30_001, 16), (18, 30_001, 1),   # 16: 4 | 17: 8
    (9, 7_456_540, 2), (9, 7_456_541, 5),  # cached | streaming stores
])
def test_broadcast_launch_form_edges(oracle, p, n, src):
    if n > 7_000_000:
        assert (p * n * 4 > 256 << 20) == (n % 2 == 1)
    host = _vals(p, n, 610 + p, False, oracle)
    bufs = [to_dev(h) for h in host]
    ddp.broadcast_sim(bufs, src=src)
    torch.cuda.synchronize()
    want, _ = oracle.broadcast(host, src)
    for r in range(p):
        assert_bits_equal(to_host(bufs[r]), want[r], f"rank {r}")


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("p,C", [(5, 10_007), (9, 10_007), (17, 3_001)])
def test_allgather_launch_form_edges(oracle, p, C, in_place):
    """In place a source skips its own rank (p - 1 destinations), out of
    place it does not (p): at 5, 9 and 17 ranks the two take different
    wave counts."""
    host = _vals(p, C, 520 + p, False, oracle)
    outs = [torch.full((p * C,), 7.0, dtype=torch.float32, device="cuda") for _ in range(p)]
    if in_place:
        ins = [outs[r][r * C:(r + 1) * C] for r in range(p)]
        for r in range(p):
            ins[r].copy_(to_dev(host[r]))
    else:
        ins = [to_dev(h) for h in host]
    ddp.allgather_sim(ins, outs)
    torch.cuda.synchronize()
    want, _ = oracle.allgather(host)
    for r in range(p):
        assert_bits_equal(to_host(outs[r]), want[r], f"rank {r}")
