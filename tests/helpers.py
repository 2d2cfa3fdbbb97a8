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
