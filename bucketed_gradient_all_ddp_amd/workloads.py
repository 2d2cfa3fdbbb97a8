"""Seeded synthetic workloads: gradient shapes, sizes and values.

This module is the only code that both the HIP path and the CPU oracle use.
It holds none of the method's arithmetic (no bucketing, no chunking, no
reduction, no averaging): only parameter shapes, seeds and random draws.

Workloads (the pages name no dataset; all inputs are synthetic):
  - "ragged ring": one fp32 tensor of 1,000,003 elements per rank at p=4
    (not divisible by p), values N(0,1), plus a 10-parameter plan whose sizes
    grow geometrically from 1K to 4M elements.
  - "gpt2-small": the 148 gradients of a GPT-2-small-shaped model in
    registration order, values N(0, 1e-3), p=8, fp32.
  - "llama-7b": the 291 gradients of a Llama-7B-shaped model, values
    N(0, 1e-4) drawn in fp32 and rounded to bf16, p=8.
  - "latency regime": 20,000 fp32 tensors with sizes log-uniform in
    [64, 65536] elements (numpy default_rng(4)), N(0,1), p=64.
  - "cost-model shape": one 2^29-element fp32 tensor per rank (2 GiB), p=64,
    N(0,1), per-rank token counts uniform in [10, 10000].

Bucket caps follow the pages' defaults: 25 MiB buckets and a 1 MiB first
bucket ("PyTorch DDP Deep Dive", Part 1; "Collective Ops From Scratch",
bucketing pattern).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

MiB = 1024 * 1024
BUCKET_CAP_BYTES = 25 * MiB
FIRST_BUCKET_CAP_BYTES = 1 * MiB

Shape = Tuple[int, ...]


def numel(shape: Sequence[int]) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


# ---------------------------------------------------------------------------
# Parameter shapes (registration order)
# ---------------------------------------------------------------------------

def geometric_sizes(count: int = 10, smallest: int = 1024,
                    ratio_total: int = 4096) -> List[int]:
    """round(smallest * ratio_total^(k/(count-1))), k = 0..count-1."""
    return [int(round(smallest * ratio_total ** (k / (count - 1))))
            for k in range(count)]


def gpt2_small_params(n_layer: int = 12, d: int = 768, vocab: int = 50257,
                      ctx: int = 1024) -> List[Tuple[str, Shape]]:
    """GPT-2 small parameter shapes in module registration order (148)."""
    out: List[Tuple[str, Shape]] = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(n_layer):
        h = f"h{i}"
        out += [
            (f"{h}.ln_1.weight", (d,)), (f"{h}.ln_1.bias", (d,)),
            (f"{h}.attn.c_attn.weight", (d, 3 * d)), (f"{h}.attn.c_attn.bias", (3 * d,)),
            (f"{h}.attn.c_proj.weight", (d, d)), (f"{h}.attn.c_proj.bias", (d,)),
            (f"{h}.ln_2.weight", (d,)), (f"{h}.ln_2.bias", (d,)),
            (f"{h}.mlp.c_fc.weight", (d, 4 * d)), (f"{h}.mlp.c_fc.bias", (4 * d,)),
            (f"{h}.mlp.c_proj.weight", (4 * d, d)), (f"{h}.mlp.c_proj.bias", (d,)),
        ]
    out += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return out


def llama7b_params(n_layer: int = 32, d: int = 4096, ffn: int = 11008,
                   vocab: int = 32000) -> List[Tuple[str, Shape]]:
    """Llama-7B parameter shapes in module registration order (291)."""
    out: List[Tuple[str, Shape]] = [("embed_tokens", (vocab, d))]
    for i in range(n_layer):
        l = f"layers.{i}"
        out += [
            (f"{l}.q_proj", (d, d)), (f"{l}.k_proj", (d, d)),
            (f"{l}.v_proj", (d, d)), (f"{l}.o_proj", (d, d)),
            (f"{l}.gate_proj", (ffn, d)), (f"{l}.up_proj", (ffn, d)),
            (f"{l}.down_proj", (d, ffn)),
            (f"{l}.input_layernorm", (d,)), (f"{l}.post_attention_layernorm", (d,)),
        ]
    out += [("norm", (d,)), ("lm_head", (vocab, d))]
    return out


def latency_regime_sizes(count: int = 20000, lo: int = 64, hi: int = 65536,
                         seed: int = 4) -> List[int]:
    """Sizes rint(exp(U(ln lo, ln hi))) from numpy default_rng(seed)."""
    rng = np.random.default_rng(seed)
    s = np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), count)))
    return [int(v) for v in s.astype(np.int64)]


def token_counts(p: int, seed: int = 5, lo: int = 10, hi: int = 10000) -> List[int]:
    """Per-rank token counts, uniform integers in [lo, hi] inclusive."""
    rng = np.random.default_rng([seed, 0x70C])
    return [int(v) for v in rng.integers(lo, hi + 1, size=p)]


# ---------------------------------------------------------------------------
# Values
# ---------------------------------------------------------------------------

def rank_seed(seed: int, rank: int, stream: int = 0) -> int:
    """Distinct 63-bit seed per (workload seed, rank, stream)."""
    x = (seed * 0x9E3779B97F4A7C15 + rank * 0xBF58476D1CE4E5B9
         + stream * 0x94D049BB133111EB + 0x2545F4914F6CDD1D)
    return x & 0x7FFFFFFFFFFFFFFF


def normal_np(n: int, sigma: float, seed: int, rank: int, stream: int = 0
              ) -> np.ndarray:
    """CPU draw: n fp32 values N(0, sigma^2) for one rank."""
    rng = np.random.default_rng(rank_seed(seed, rank, stream))
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def normal_torch(n: int, sigma: float, seed: int, rank: int, device,
                 dtype=None, stream: int = 0, out=None):
    """Device draw with torch's generator for that device: n values
    N(0, sigma^2), drawn in fp32 and then cast to `dtype` (fp32 or bf16,
    the cast rounding to nearest even). Deterministic per (seed, rank,
    stream, device type)."""
    import torch

    dtype = dtype or torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(rank_seed(seed, rank, stream))
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    if out is not None:
        out.copy_(x)
        return out
    return x if dtype == torch.float32 else x.to(dtype)


def integer_valued_np(n: int, seed: int, rank: int, bound: int = 1024
                      ) -> np.ndarray:
    """fp32 values that are integers in [-bound, bound]."""
    rng = np.random.default_rng(rank_seed(seed, rank, 7))
    return rng.integers(-bound, bound + 1, size=n).astype(np.float32)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

WORKLOADS = {
    "ragged-ring-p4": dict(p=4, n=1_000_003, sigma=1.0, seed=1, dtype="f32",
                           plan_sizes=geometric_sizes()),
    "gpt2-small-p8": dict(p=8, sigma=1e-3, seed=2, dtype="f32",
                          params=gpt2_small_params(), avg="world"),
    "llama7b-bf16-p8": dict(p=8, sigma=1e-4, seed=3, dtype="bf16",
                            params=llama7b_params(), avg="world"),
    "latency-p64": dict(p=64, sigma=1.0, seed=4, dtype="f32",
                        sizes=latency_regime_sizes(), avg="world"),
    "cost-model-p64": dict(p=64, n=1 << 29, sigma=1.0, seed=5, dtype="f32",
                           avg="tokens"),
    # the same operations on 8 ranks of 1 GiB (the headline's rank count with
    # flat buffers well past the Infinity Cache)
    "collectives-p8": dict(p=8, n=1 << 28, sigma=1.0, seed=6, dtype="f32",
                           avg="tokens"),
}
