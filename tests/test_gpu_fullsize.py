"""GPU parity at the workloads' full sizes.

- GPT-2 small (124M fp32 per rank, p=8): every element of every rank is
  compared with the oracle's flatten -> literal ring -> unflatten, for the
  in-place bucket all-reduce (one launch for all buckets, one per bucket,
  and the reducer's capped launches), the three-kernel path and the
  ring-step path.
- Llama-7B (6.7G bf16 per rank, p=8, 108 GB resident), the latency regime
  (20,000 tensors, p=64) and the 2 GiB x 64 cost-model shape: sampled
  elements (random ones plus every chunk's first and last element) are
  checked bit for bit against the oracle's per-element ring fold, whose
  equality with the literal ring is pinned on the CPU; every rank must hold
  identical bits at every sample.
Inputs are drawn on the GPU and the sampled inputs copied to the host before
any kernel of the library runs.
"""
import bisect

import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_host

pytestmark = pytest.mark.gpu

GiB = 1 << 30


def _say(msg):
    print(f"[fullsize] {msg}", flush=True)


def _need(nbytes):
    free, total = torch.cuda.mem_get_info()
    if total < nbytes * 1.1:
        pytest.skip(f"needs {nbytes / GiB:.0f} GiB of device memory")


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _arenas(p, sizes, sigma, seed, dtype, align=64):
    """One arena per rank, parameters in registration order, each at an
    `align`-element boundary. Drawn in fp32 pieces and cast."""
    offs, off = [], 0
    for n in sizes:
        offs.append(off)
        off += (n + align - 1) // align * align
    arenas = []
    piece = 1 << 28
    for r in range(p):
        a = torch.empty(off, dtype=dtype, device="cuda")
        for k, lo in enumerate(range(0, off, piece)):
            hi = min(off, lo + piece)
            a[lo:hi].copy_(W.normal_torch(hi - lo, sigma, seed, r, "cuda", stream=k))
        arenas.append(a)
    grads = [[a[o:o + n] for o, n in zip(offs, sizes)] for a in arenas]
    return arenas, offs, grads


def _samples(n, p, k, rng):
    """k random indices of [0, n) plus the first and last element of every
    chunk of ceil(n/p)."""
    C = -(-n // p)
    edges = [v for c in range(p) for v in (c * C, min((c + 1) * C, n) - 1) if c * C < n]
    idx = np.concatenate([rng.integers(0, n, size=k), np.array(edges, dtype=np.int64)])
    return np.unique(idx)


def _gather(bufs, idx_np):
    idx = torch.from_numpy(idx_np).to("cuda")
    return np.stack([to_host(b[idx]) for b in bufs], axis=1)


class _BucketIndex:
    """Maps (bucket, flat index) to the arena index of the element."""

    def __init__(self, oplan, offs):
        self.oplan, self.offs = oplan, offs
        self.starts, self.params = [], []
        for b in range(oplan.num_buckets):
            ps = oplan.bucket_params(b)
            self.params.append(ps)
            self.starts.append([int(oplan.offset[i]) for i in ps])

    def arena_index(self, b, flat):
        out = np.empty(len(flat), dtype=np.int64)
        for k, i in enumerate(flat):
            j = bisect.bisect_right(self.starts[b], int(i)) - 1
            prm = self.params[b][j]
            out[k] = self.offs[prm] + int(i) - self.starts[b][j]
        return out


# ---------------------------------------------------------------------------

def test_gpt2_small_full_compare(oracle):
    cfg = W.WORKLOADS["gpt2-small-p8"]
    p = cfg["p"]
    sizes = [W.numel(s) for _, s in cfg["params"]]
    _need(3 * p * sum(sizes) * 4)
    plan = ddp.ddp_bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    plan.upload().upload_segments(p)
    oplan = oracle.bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    assert plan.buckets() == oplan.buckets() and plan.num_buckets == 13
    arenas, offs, grads = _arenas(p, sizes, cfg["sigma"], cfg["seed"], torch.float32)
    _say("gpt2: inputs drawn; running the oracle")
    host = [[to_host(g) for g in rank] for rank in grads]
    want = [[g.copy() for g in rank] for rank in host]
    for b in range(oplan.num_buckets):
        flats = [oracle.flatten(want[r], oplan, b) for r in range(p)]
        red, _ = oracle.ring_allreduce(flats, avg="world", want_log=False)
        for r in range(p):
            oracle.unflatten(red[r], oplan, b, want[r])
        del flats, red
    table = ddp.grad_pointer_table(grads)
    for path in ("batched", "inplace", "reducer-capped", "copy-fused", "copy-ring"):
        _say(f"gpt2: {path}")
        for r in range(p):
            for i, g in enumerate(grads[r]):
                g.copy_(torch.from_numpy(host[r][i]))
        if path == "batched":
            # the benchmark's headline launch: every bucket in one dispatch
            ddp.ddp_allreduce_buckets(plan, 0, plan.num_buckets, table, p, avg="world")
        if path == "reducer-capped":
            # the overlap workload's form: the reducer on its own stream, each
            # launch capped at 1,024 workgroups, parameters marked in reverse
            torch.cuda.synchronize()
            comm = torch.cuda.Stream()
            reducer = ddp.Reducer(plan, p, table, avg="world", comm_stream=comm)
            reducer.set_max_workgroups(1024)
            reducer.prepare()
            for i in reversed(range(len(sizes))):
                reducer.mark_ready(i)
            reducer.finalize(torch.cuda.current_stream())
        for b in range(plan.num_buckets if path in ("inplace", "copy-fused", "copy-ring") else 0):
            if path == "inplace":
                ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
            else:
                bufs = [torch.empty(plan.bucket_numel(b), device="cuda") for _ in range(p)]
                ddp.ddp_flatten(plan, b, table, bufs)
                ddp.ring_allreduce_sim(bufs, avg="world", algo=path.split("-")[1])
                ddp.ddp_unflatten(plan, b, bufs, table)
                del bufs
        torch.cuda.synchronize()
        for r in range(p):
            got = to_host(arenas[r])
            for i, n in enumerate(sizes):
                assert_bits_equal(got[offs[i]:offs[i] + n], want[r][i], f"{path} rank {r} param {i}")
    del arenas, grads, host, want
    _free()


def test_llama7b_bf16_sampled(oracle):
    cfg = W.WORKLOADS["llama7b-bf16-p8"]
    p = cfg["p"]
    sizes = [W.numel(s) for _, s in cfg["params"]]
    _need(p * sum(sizes) * 2 + 8 * GiB)
    plan = ddp.ddp_bucket_plan(sizes, 2, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    plan.upload().upload_segments(p)
    oplan = oracle.bucket_plan(sizes, 2, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    assert plan.num_buckets == 226 and plan.buckets() == oplan.buckets()
    arenas, offs, grads = _arenas(p, sizes, cfg["sigma"], cfg["seed"], torch.bfloat16)
    _say("llama7b: inputs drawn (%.1f GB)" % (p * sum(sizes) * 2 / 1e9))
    table = ddp.grad_pointer_table(grads)
    index = _BucketIndex(oplan, offs)
    rng = np.random.default_rng(3)
    picks = []
    for b in range(plan.num_buckets):
        flat = _samples(plan.bucket_numel(b), p, 256, rng)
        ai = index.arena_index(b, flat)
        picks.append((b, flat, ai, _gather(arenas, ai)))
    # whole buckets, every element: both 262 MB buckets (the head, filled
    # first, and the embedding, filled last), the 90 MB bucket of four
    # parameters that mixes the RMSNorm weights with a projection, and a
    # 33.5 MB attention bucket
    whole_buckets = (0, 1, 4, plan.num_buckets - 1)
    assert [plan.bucket_numel(b) * 2 for b in (0, 1, 4)] == [262_144_000, 90_202_112, 33_554_432]
    whole = {}
    for b in whole_buckets:
        whole[b] = [oracle.flatten(_host_params(grads[r], oplan.bucket_params(b)), oplan, b)
                    for r in range(p)]
    _say("llama7b: samples and %d whole buckets taken; all-reducing 226 buckets"
         % len(whole_buckets))
    # the first half as one launch (the batched form the benchmark also
    # times), the rest one launch per bucket
    half = plan.num_buckets // 2
    ddp.ddp_allreduce_buckets(plan, 0, half, table, p, avg="world")
    for b in range(half, plan.num_buckets):
        ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
    torch.cuda.synchronize()
    _say("llama7b: checking")
    for b, flat, ai, vals in picks:
        want = oracle.allreduce_at(vals, flat, plan.bucket_numel(b), avg="world")
        got = _gather(arenas, ai)
        for r in range(p):
            assert_bits_equal(got[:, r], want, f"bucket {b} rank {r}")
        s = oracle.bf16_to_f32(vals).astype(np.float64).sum(1) / p
        y = oracle.bf16_to_f32(want).astype(np.float64)
        scale = np.abs(oracle.bf16_to_f32(vals)).astype(np.float64).sum(1) / p
        assert np.all(np.abs(y - s) <= 1e-2 * np.abs(s) + (p - 1) * 2.0 ** -24 * scale + 1e-45)
    for b in whole_buckets:
        want, _ = oracle.ring_allreduce(whole[b], avg="world", want_log=False)
        for r in range(p):
            got = oracle.flatten(_host_params(grads[r], oplan.bucket_params(b)), oplan, b)
            assert_bits_equal(got, want[r], f"whole bucket {b} rank {r}")
        # the stated bound against an fp64 sum, norm-wise per bucket
        s = np.zeros(want[0].size, dtype=np.float64)
        for r in range(p):
            s += oracle.bf16_to_f32(whole[b][r])
        s /= p
        y = oracle.bf16_to_f32(want[0]).astype(np.float64)
        assert np.linalg.norm(y - s) <= 1e-2 * np.linalg.norm(s)
        _say("llama7b: whole bucket %d (%d elements x %d ranks) matches" % (b, want[0].size, p))
        del want, s, y
        whole[b] = None
    del arenas, grads
    _free()


def _host_params(rank_grads, params):
    """One rank's gradients of `params` on the host (bf16 as uint16 bit
    patterns), indexed by parameter, None elsewhere: the oracle's flatten
    input."""
    out = [None] * len(rank_grads)
    for i in params:
        out[i] = to_host(rank_grads[i])
    return out


def test_latency_regime_per_tensor_and_bucketed(oracle):
    cfg = W.WORKLOADS["latency-p64"]
    p = cfg["p"]
    sizes = cfg["sizes"]
    _need(p * sum(sizes) * 4 + 4 * GiB)
    rng = np.random.default_rng(4)
    # per-tensor: each tensor is its own all-reduce (own padding and chunks)
    arenas, offs, grads = _arenas(p, sizes, 1.0, cfg["seed"], torch.float32)
    check = sorted(set(rng.choice(len(sizes), 60, replace=False).tolist())
                   | {int(np.argmin(sizes)), int(np.argmax(sizes))})
    before = {i: [to_host(grads[r][i]) for r in range(p)] for i in check}
    _say("latency: per-tensor all-reduce of 20,000 tensors")
    for i in range(len(sizes)):
        ddp.ring_allreduce_sim([grads[r][i] for r in range(p)], avg="world")
    torch.cuda.synchronize()
    for i in check:
        want, _ = oracle.ring_allreduce(before[i], avg="world", want_log=False)
        for r in range(p):
            assert_bits_equal(to_host(grads[r][i]), want[r], f"tensor {i} rank {r}")
    del arenas, grads, before
    _free()
    # bucketed, in place
    _say("latency: bucketed")
    plan = ddp.ddp_bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    plan.upload_segments(p)
    oplan = oracle.bucket_plan(sizes, 4, W.BUCKET_CAP_BYTES, W.FIRST_BUCKET_CAP_BYTES)
    assert plan.buckets() == oplan.buckets()
    arenas, offs, grads = _arenas(p, sizes, 1.0, cfg["seed"] + 100, torch.float32)
    table = ddp.grad_pointer_table(grads)
    index = _BucketIndex(oplan, offs)
    picks = []
    for b in range(plan.num_buckets):
        flat = _samples(plan.bucket_numel(b), p, 512, rng)
        ai = index.arena_index(b, flat)
        picks.append((b, flat, ai, _gather(arenas, ai)))
    for b in range(plan.num_buckets):
        ddp.ddp_allreduce_bucket(plan, b, table, p, avg="world")
    torch.cuda.synchronize()
    for b, flat, ai, vals in picks:
        want = oracle.allreduce_at(vals, flat, plan.bucket_numel(b), avg="world")
        got = _gather(arenas, ai)
        for r in range(p):
            assert_bits_equal(got[:, r], want, f"bucket {b} rank {r}")
    # the same 30 buckets as one launch, on the results as new inputs
    picks = [(b, flat, ai, _gather(arenas, ai)) for b, flat, ai, _ in picks]
    _say("latency: bucketed, one launch for all buckets")
    ddp.ddp_allreduce_buckets(plan, 0, plan.num_buckets, table, p, avg="world")
    torch.cuda.synchronize()
    for b, flat, ai, vals in picks:
        want = oracle.allreduce_at(vals, flat, plan.bucket_numel(b), avg="world")
        got = _gather(arenas, ai)
        for r in range(p):
            assert_bits_equal(got[:, r], want, f"one launch: bucket {b} rank {r}")
    # the per-tensor arithmetic in one launch: caps of 0 bytes, every tensor
    # its own bucket
    _say("latency: per-tensor, one launch for all tensors")
    tplan = ddp.ddp_bucket_plan(sizes, 4, 0, 0).upload_segments(p)
    before = {i: [to_host(grads[r][i]) for r in range(p)] for i in check}
    ddp.ddp_allreduce_buckets(tplan, 0, tplan.num_buckets, table, p, avg="world")
    torch.cuda.synchronize()
    for i in check:
        want, _ = oracle.ring_allreduce(before[i], avg="world", want_log=False)
        for r in range(p):
            assert_bits_equal(to_host(grads[r][i]), want[r], f"one launch: tensor {i} rank {r}")
    del arenas, grads, tplan
    _free()


def test_cost_model_shape_p64_2gib(oracle):
    cfg = W.WORKLOADS["cost-model-p64"]
    p, n = cfg["p"], cfg["n"]
    _need(p * n * 4 + 4 * GiB)
    tokens = W.token_counts(p, cfg["seed"])
    bufs = [W.normal_torch(n, 1.0, cfg["seed"], r, "cuda") for r in range(p)]
    rng = np.random.default_rng(5)
    C = n // p
    idx = _samples(n, p, 4096, rng)
    vals = _gather(bufs, idx)

    # a whole window across the end of chunk 31 and the start of chunk 32,
    # every element
    lo = 32 * C - (1 << 19)
    window = np.arange(lo, lo + (1 << 20), dtype=np.int64)
    wvals = np.stack([to_host(b[lo:lo + (1 << 20)]) for b in bufs], axis=1)

    # token-weighted all-reduce, fused
    _say("cost-model shape: all-reduce of 64 x 2 GiB")
    ddp.ring_allreduce_sim(bufs, avg="tokens", tokens=tokens)
    torch.cuda.synchronize()
    want = oracle.allreduce_at(vals, idx, n, avg="tokens", tokens=tokens)
    got = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got[:, r], want, f"all-reduce rank {r}")
    want = oracle.allreduce_at(wvals, window, n, avg="tokens", tokens=tokens)
    for r in range(p):
        assert_bits_equal(to_host(bufs[r][lo:lo + (1 << 20)]), want, f"window rank {r}")
    # every element of every rank: all ranks hold the same bits afterwards
    for r in range(1, p):
        assert torch.equal(bufs[r].view(torch.int32), bufs[0].view(torch.int32)), f"rank {r}"
    del wvals

    # standalone reduce-scatter (pre-rotated), on fresh values
    for r in range(p):
        W.normal_torch(n, 1.0, cfg["seed"] + 1, r, "cuda", out=bufs[r])
    vals = _gather(bufs, idx)
    outs = [torch.empty(C, device="cuda") for _ in range(p)]
    _say("cost-model shape: reduce-scatter, all-gather, broadcast")
    ddp.reduce_scatter_sim(bufs, outs, avg="tokens", tokens=tokens)
    torch.cuda.synchronize()
    want = oracle.reduce_scatter_at(vals, idx, n, avg="tokens", tokens=tokens)
    for k, i in enumerate(idx):
        owner, pos = int(i) // C, int(i) % C
        got = to_host(outs[owner][pos:pos + 1])
        assert_bits_equal(got, want[k:k + 1], f"reduce-scatter element {i}")

    # all-gather in place: shard r of rank r's buffer is its contribution
    for r in range(p):
        bufs[r][r * C:(r + 1) * C].copy_(outs[r])
    shards = [bufs[r][r * C:(r + 1) * C] for r in range(p)]
    ddp.allgather_sim(shards, bufs)
    torch.cuda.synchronize()
    got = _gather(bufs, idx)
    for k, i in enumerate(idx):
        owner, pos = int(i) // C, int(i) % C
        expect = to_host(outs[owner][pos:pos + 1])[0]
        assert np.all(got[k].view(np.uint32) == np.float32(expect).view(np.uint32))

    # broadcast from rank 0 of fresh values
    W.normal_torch(n, 1.0, cfg["seed"] + 2, 0, "cuda", out=bufs[0])
    src = _gather(bufs[:1], idx)[:, 0]
    ddp.broadcast_sim(bufs, src=0)
    torch.cuda.synchronize()
    got = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got[:, r], src, f"broadcast rank {r}")

    # the token-weighted all-reduce under each logarithmic schedule, fused,
    # each on fresh values
    for k, schedule in enumerate(("recursive_doubling", "rabenseifner", "tree")):
        for r in range(p):
            W.normal_torch(n, 1.0, cfg["seed"] + 3 + k, r, "cuda", out=bufs[r])
        vals = _gather(bufs, idx)
        _say(f"cost-model shape: {schedule} all-reduce of 64 x 2 GiB")
        ddp.allreduce_sim(bufs, schedule, False, avg="tokens", tokens=tokens)
        torch.cuda.synchronize()
        want = oracle.tree_allreduce_at(vals, schedule, avg="tokens", tokens=tokens)
        got = _gather(bufs, idx)
        for r in range(p):
            assert_bits_equal(got[:, r], want, f"{schedule} rank {r}")
    del bufs, outs
    _free()


def test_beyond_two_to_the_31_elements(oracle):
    """Index arithmetic past 32 bits: p = 2 buffers of 2^31 + 7 fp32 elements
    (8 GiB each) through the fused ring all-reduce, then the same elements as
    one parameter of a bucket plan through the in-place bucket all-reduce,
    the fused tree all-reduce and the coalesced broadcast; sampled elements
    (random ones, every chunk's ends and the last elements) against the
    oracle."""
    p, n = 2, (1 << 31) + 7
    _need(p * n * 4 + 4 * GiB)
    rng = np.random.default_rng(11)
    bufs = [W.normal_torch(n, 1.0, 31, r, "cuda") for r in range(p)]
    idx = np.unique(np.concatenate([_samples(n, p, 2048, rng),
                                    np.arange(n - 40, n, dtype=np.int64)]))
    vals = _gather(bufs, idx)
    _say("2^31+7: fused ring all-reduce")
    ddp.ring_allreduce_sim(bufs, avg="world")
    torch.cuda.synchronize()
    want = oracle.allreduce_at(vals, idx, n, avg="world")
    got = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got[:, r], want, f"ring rank {r}")
    # the results are the next inputs: one parameter, one bucket
    vals2 = got.copy()
    plan = ddp.ddp_bucket_plan([n], 4, 25 << 20, 1 << 20).upload_segments(p)
    table = ddp.grad_pointer_table([[b] for b in bufs])
    _say("2^31+7: in-place bucket all-reduce")
    ddp.ddp_allreduce_buckets(plan, 0, 1, table, p, avg="none")
    torch.cuda.synchronize()
    want2 = oracle.allreduce_at(vals2, idx, n, avg="none")
    got2 = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got2[:, r], want2, f"bucket rank {r}")
    # the tree all-reduce (fused) and the coalesced broadcast on the same
    # buffers
    vals3 = got2.copy()
    _say("2^31+7: tree all-reduce")
    ddp.allreduce_sim(bufs, "tree", False, avg="world")
    torch.cuda.synchronize()
    want3 = oracle.tree_allreduce_at(vals3, "tree", avg="world")
    got3 = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got3[:, r], want3, f"tree rank {r}")
    bufs[1].add_(1.0)  # make the ranks differ again
    _say("2^31+7: coalesced broadcast from rank 1")
    bplan = ddp.ddp_coalesce_plan([n], 4, 1 << 40).upload()
    ddp.ddp_broadcast_coalesced(bplan, table, p, 1)
    torch.cuda.synchronize()
    got4 = _gather(bufs, idx)
    assert np.array_equal(got4[:, 0].view(np.uint32), got4[:, 1].view(np.uint32))
    assert np.array_equal(got4[:, 1], (got3[:, 1] + np.float32(1.0)).astype(np.float32))
    del bufs
    _free()


def test_beyond_two_to_the_31_elements_many_ranks(oracle):
    """Index arithmetic past 32 bits in the kernels that split a tile's ranks
    over waves: p = 17 bf16 buffers of 17 * 126,322,576 elements (just over
    2^31, 4 GiB each) through the fused ring all-reduce, the reduce-scatter
    and the fused tree all-reduce, each on fresh values; sampled elements
    (random ones, every chunk's ends and the last elements) against the
    oracle."""
    p, C = 17, 126_322_576
    n = p * C
    assert n > 1 << 31
    _need(p * n * 2 + p * C * 2 + 8 * GiB)
    rng = np.random.default_rng(12)
    bufs = [W.normal_torch(n, 1.0, 41, r, "cuda", dtype=torch.bfloat16) for r in range(p)]
    idx = np.unique(np.concatenate([_samples(n, p, 2048, rng),
                                    np.arange(n - 40, n, dtype=np.int64)]))
    vals = _gather(bufs, idx)
    assert vals.dtype == np.uint16
    _say("17 x (2^31+): fused ring all-reduce, bf16")
    ddp.ring_allreduce_sim(bufs, avg="world")
    torch.cuda.synchronize()
    want = oracle.allreduce_at(vals, idx, n, avg="world")
    got = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got[:, r], want, f"ring rank {r}")

    for r in range(p):
        W.normal_torch(n, 1.0, 42, r, "cuda", dtype=torch.bfloat16, out=bufs[r])
    vals = _gather(bufs, idx)
    outs = [torch.empty(C, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    _say("17 x (2^31+): reduce-scatter, bf16")
    ddp.reduce_scatter_sim(bufs, outs, avg="world")
    torch.cuda.synchronize()
    want = oracle.reduce_scatter_at(vals, idx, n, avg="world")
    owner, pos = idx // C, idx % C
    got = np.array([to_host(outs[int(o)][int(j):int(j) + 1])[0] for o, j in zip(owner, pos)],
                   dtype=np.uint16)
    assert_bits_equal(got, want, "reduce-scatter")
    del outs

    for r in range(p):
        W.normal_torch(n, 1.0, 43, r, "cuda", dtype=torch.bfloat16, out=bufs[r])
    vals = _gather(bufs, idx)
    _say("17 x (2^31+): tree all-reduce, bf16")
    ddp.allreduce_sim(bufs, "tree", False, avg="world")
    torch.cuda.synchronize()
    want = oracle.tree_allreduce_at(vals, "tree", avg="world")
    got = _gather(bufs, idx)
    for r in range(p):
        assert_bits_equal(got[:, r], want, f"tree rank {r}")
    del bufs
    _free()
