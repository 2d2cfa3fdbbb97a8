"""Pin token-weighted and world averaging on a linear model.

"Data parallelism", section "Why averaging gradients is exactly large-batch
training": the full-batch gradient equals the average of per-rank gradients
when shards are equal; with uneven token counts, sum token losses per rank,
sum the counts across ranks and divide once. Per-token loss here is
(w.x - y)^2 / 2, so the gradient of a sum of token losses is
sum_t (w.x_t - y_t) x_t.
"""
import numpy as np
import pytest

D = 16


def _shards(counts, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(D).astype(np.float32)
    xs = [rng.standard_normal((c, D)).astype(np.float32) for c in counts]
    ys = [rng.standard_normal(c).astype(np.float32) for c in counts]
    return w, xs, ys


def _grad_sum(w, x, y):
    return ((x @ w - y)[:, None] * x).sum(0).astype(np.float32)


def _full_mean_fp64(w, xs, ys):
    x = np.concatenate(xs).astype(np.float64)
    y = np.concatenate(ys).astype(np.float64)
    return ((x @ w.astype(np.float64) - y)[:, None] * x).mean(0)


@pytest.mark.parametrize("counts", [[3, 50, 200, 1000], [10, 10000, 17, 999, 5, 64, 2, 300]])
def test_token_average_equals_full_batch(oracle, counts):
    w, xs, ys = _shards(counts, seed=len(counts))
    grads = [_grad_sum(w, x, y) for x, y in zip(xs, ys)]
    out, _ = oracle.ring_allreduce(grads, avg="tokens", tokens=counts)
    ref = _full_mean_fp64(w, xs, ys)
    assert np.max(np.abs(out[0] - ref)) <= 1e-5 * np.max(np.abs(ref))
    # negative control: averaging per-rank means over-weights small ranks
    means = [g / np.float32(c) for g, c in zip(grads, counts)]
    wrong, _ = oracle.ring_allreduce(means, avg="world")
    assert np.max(np.abs(wrong[0] - ref)) > 1e-2 * np.max(np.abs(ref))


def test_world_average_of_equal_shards(oracle):
    counts = [256] * 8
    w, xs, ys = _shards(counts, seed=99)
    means = [_grad_sum(w, x, y) / np.float32(c) for x, y, c in zip(xs, ys, counts)]
    out, _ = oracle.ring_allreduce(means, avg="world")
    ref = _full_mean_fp64(w, xs, ys)
    assert np.max(np.abs(out[0] - ref)) <= 1e-5 * np.max(np.abs(ref))
