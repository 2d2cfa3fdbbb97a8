"""Helpers shared by the GPU parity tests (marshalling only)."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev(arr: np.ndarray) -> torch.Tensor:
    """numpy float32 -> cuda float32; numpy uint16 (bf16 bits) -> cuda bfloat16."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16).copy()).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> numpy (bf16 comes back as uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what=""):
    g, w = bits(got), bits(want)
    if not np.array_equal(g, w):
        bad = np.nonzero(g != w)[0]
        raise AssertionError(
            f"{what}: {bad.size} of {g.size} elements differ; first at {bad[:5].tolist()}: "
            f"got {got[bad[:3]].tolist()} want {want[bad[:3]].tolist()}")


def tokens_for(p: int, seed: int = 0):
    rng = np.random.default_rng(seed + 17 * p)
    return [int(v) for v in rng.integers(10, 10001, size=p)]


def make_grads(p, sizes, seed, bf16, oracle, layout="aligned"):
    """Per-rank gradients as views into one arena per rank.

    layout: "aligned" (every view starts on a 32-byte boundary), "odd" (views
    at odd element offsets, the same on every rank) or "mixed" (each rank
    shifted differently, so ranks disagree on the 16-byte phase)."""
    from bucketed_gradient_all_ddp_amd import workloads as W

    host = [[W.normal_np(n, 1.0, seed, r, stream=i) for i, n in enumerate(sizes)]
            for r in range(p)]
    if bf16:
        host = [[oracle.f32_to_bf16(g) for g in rank] for rank in host]
    dt = torch.bfloat16 if bf16 else torch.float32
    grads = []
    for r in range(p):
        total = sum(sizes) + 9 * len(sizes) + 16
        arena = torch.zeros(total, dtype=dt, device="cuda")
        off = {"aligned": 0, "odd": 1, "mixed": r % 3 + 1}[layout]
        views = []
        for i, n in enumerate(sizes):
            if layout == "aligned":
                off = (off + 7) // 8 * 8
            v = arena[off:off + n]
            v.copy_(to_dev(host[r][i]))
            views.append(v)
            off += n + (0 if layout == "aligned" else 1)
        grads.append(views)
    return host, grads
