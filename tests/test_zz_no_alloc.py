"""GPU: ring_allreduce_sim_noalloc (the entry point for callers that cannot
allocate) leaves exactly the bits of ring_allreduce_sim on the same inputs,
with its bf16 ring workspace in the library's per-GPU scratch array: two
calls in a row, the second smaller than the first, so the second runs on
what the first left in the array."""
import ctypes

import numpy as np
import pytest
import torch

import bucketed_gradient_all_ddp_amd as ddp
from bucketed_gradient_all_ddp_amd import workloads as W
from helpers import assert_bits_equal, to_dev, to_host, tokens_for

pytestmark = pytest.mark.gpu


def _inputs(oracle, p, n, seed, bf16):
    host = [W.normal_np(n, 1.0, seed, r) for r in range(p)]
    if bf16:
        host = [oracle.f32_to_bf16(h) for h in host]
    return host


def _both(host, p, avg, tokens, algo, dtype_bytes):
    """The same inputs through ring_allreduce_sim (with a workspace tensor)
    and through ring_allreduce_sim_noalloc (C ABI, no workspace)."""
    L = ddp.load_library()
    a = [to_dev(h) for h in host]
    b = [to_dev(h) for h in host]
    n = host[0].size
    code = ddp.DTYPE_BF16 if dtype_bytes == 2 else ddp.DTYPE_F32
    need = ddp.ring_allreduce_sim_workspace(p, n, code, algo)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda") if need else None
    ddp.ring_allreduce_sim(a, avg=avg, tokens=tokens, algo=algo, workspace=ws)
    ptrs = (ctypes.c_void_p * p)(*[t.data_ptr() for t in b])
    tok = (ctypes.c_int64 * p)(*tokens) if tokens is not None else None
    st = ddp.CommStats()
    stream = torch.cuda.current_stream().cuda_stream
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    rc = L.ring_allreduce_sim_noalloc(ptrs, p, n, code, ddp.AVG[avg], tok, ddp.ALGO[algo],
                                      stream, ctypes.byref(st))
    assert rc == 0, L.ddp_last_error()
    assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before
    torch.cuda.synchronize()
    return a, b, st, need


@pytest.mark.parametrize("avg", ["world", "tokens"])
@pytest.mark.parametrize("p", [8, 5])
def test_noalloc_bf16_ring_twice_second_smaller(oracle, p, avg):
    tokens = tokens_for(p, 5) if avg == "tokens" else None
    # first call: a workspace close to the scratch array's size
    n1 = (ddp.NOALLOC_SCRATCH_BYTES // (4 * p)) - 4096 - 3
    n2 = 100_003
    for k, n in enumerate((n1, n2)):
        host = _inputs(oracle, p, n, 4200 + 10 * p + k, True)
        a, b, st, need = _both(host, p, avg, tokens, "ring", 2)
        assert 0 < need <= ddp.NOALLOC_SCRATCH_BYTES
        assert st.steps == 2 * (p - 1)
        for r in range(p):
            assert_bits_equal(to_host(b[r]), to_host(a[r]), f"call {k} n={n} rank {r}")
        if n == n2:
            want, _ = oracle.ring_allreduce(host, avg=avg, tokens=tokens, want_log=False)
            for r in range(p):
                assert_bits_equal(to_host(b[r]), want[r], f"oracle n={n} rank {r}")


@pytest.mark.parametrize("algo,bf16", [("fused", True), ("fused", False), ("ring", False)])
def test_noalloc_paths_without_workspace(oracle, algo, bf16):
    """Paths that need no workspace run with no size limit, same bits."""
    p, n = 4, 1_000_003
    host = _inputs(oracle, p, n, 4300, bf16)
    a, b, st, need = _both(host, p, "world", None, algo, 2 if bf16 else 4)
    assert need == 0
    for r in range(p):
        assert_bits_equal(to_host(b[r]), to_host(a[r]), f"rank {r}")


def test_noalloc_refuses_a_workspace_past_the_scratch_array():
    """Too large: DDP_EWORKSPACE, nothing enqueued (the buffers keep their
    values)."""
    p = 8
    n = ddp.NOALLOC_SCRATCH_BYTES // (4 * p) + 1
    bufs = [torch.full((n,), 1.0, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    with pytest.raises(ddp.DDPError, match="EWORKSPACE") as e:
        ddp.ring_allreduce_sim_noalloc(bufs, avg="none", algo="ring")
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    for t in bufs:
        assert bool((t == 1.0).all())
