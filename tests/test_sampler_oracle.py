"""Pins of the reference sampler (oracle/sampler.py).

Against the pages' worked example ("vLLM 基本原理", FlashInfer 采样器: logits
8.2 / 7.9 / 5.1 / 1.2 with temperature 0.7, top_k 50, top_p 0.9), a brute-force
re-derivation on tiny vocabularies written with plain Python loops, closed
forms (top_k = 1 and a tiny top_p give the argmax; equal logits give a
uniform draw), and the inverse distribution function (u = 0 gives the first
kept token, a uniform grid of u reproduces the probabilities).
"""
import math

import numpy as np
import pytest

from oracle import sampler


def brute(logits, t, k, p):
    """The definition with loops: temperature, top-k (ties kept), renormalise,
    top-p (mass strictly above < P), renormalise."""
    v = len(logits)
    z = [x / t for x in logits]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    keep = [True] * v
    if 0 < k < v:
        kth = sorted(z, reverse=True)[k - 1]
        keep = [z[i] >= kth for i in range(v)]
    tot = sum(w[i] for i in range(v) if keep[i])
    q = [w[i] / tot if keep[i] else 0.0 for i in range(v)]
    if p < 1:
        keep2 = []
        for i in range(v):
            above = sum(q[j] for j in range(v) if keep[j] and q[j] > q[i])
            keep2.append(keep[i] and above < p)
        tot = sum(q[i] for i in range(v) if keep2[i])
        q = [q[i] / tot if keep2[i] else 0.0 for i in range(v)]
    return q


def test_pages_worked_example():
    logits = [8.2, 7.9, 5.1, 1.2]           # 你好 / 您好 / 今天 / 苹果
    got = sampler.probabilities(logits, 0.7, 50, 0.9)
    e0, e1 = math.exp(8.2 / 0.7), math.exp(7.9 / 0.7)
    # top_k 50 keeps all four; the two leading tokens hold > 0.99 of the mass, the first
    # alone about 0.60 < 0.9, so top_p keeps exactly those two
    assert got[2] == 0 and got[3] == 0
    assert got[0] == pytest.approx(e0 / (e0 + e1), rel=1e-12)
    assert got[1] == pytest.approx(e1 / (e0 + e1), rel=1e-12)
    assert sampler.sample(logits, 0.7, 50, 0.9, 0.0) == 0
    assert sampler.sample(logits, 0.7, 50, 0.9, 0.99) == 1


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_on_tiny_vocabularies(seed):
    rng = np.random.default_rng(seed)
    v = int(rng.integers(1, 9))
    logits = [float(x) for x in np.round(rng.normal(0, 2, v), 1)]   # rounding makes ties
    t = float(rng.choice([0.3, 0.7, 1.0, 2.5]))
    k = int(rng.integers(0, v + 2))
    p = float(rng.choice([0.05, 0.5, 0.9, 0.99, 1.0]))
    np.testing.assert_allclose(sampler.probabilities(logits, t, k, p), brute(logits, t, k, p),
                               rtol=1e-12, atol=1e-15)


def test_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, 1000)
    a = int(np.argmax(x))
    for u in (0.0, 0.3, 0.999):
        assert sampler.sample(x, 0.7, 1, 1.0, u) == a          # top_k = 1
        assert sampler.sample(x, 1.0, 0, 1e-9, u) == a         # a tiny top_p
    flat = np.zeros(10)
    np.testing.assert_allclose(sampler.probabilities(flat, 1.0, 3, 1.0), np.full(10, 0.1))
    assert sampler.sample([-np.inf, np.nan, -np.inf], 1.0, 0, 1.0, 0.5) == -1
    assert sampler.sample([-np.inf, 2.0, np.nan], 1.0, 0, 1.0, 0.5) == 1
    np.testing.assert_array_equal(sampler.probabilities([np.inf, 3.0, np.inf], 1.0, 0, 1.0),
                                  [0.5, 0.0, 0.5])


def test_inverse_distribution_function():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1.5, 64)
    p = sampler.probabilities(x, 0.8, 20, 0.95)
    kept = np.nonzero(p)[0]
    assert sampler.sample(x, 0.8, 20, 0.95, 0.0) == kept[0]
    assert sampler.sample(x, 0.8, 20, 0.95, np.nextafter(1.0, 0.0)) == kept[-1]
    n = 100_000
    draws = [sampler.sample(x, 0.8, 20, 0.95, (i + 0.5) / n) for i in range(0, n, 7)]
    counts = np.bincount(draws, minlength=64) / len(draws)
    assert np.abs(counts - p).max() < 2e-3


def test_invalid_parameters():
    with pytest.raises(ValueError):
        sampler.probabilities([1.0], 0.0, 0, 1.0)
    with pytest.raises(ValueError):
        sampler.probabilities([1.0], 1.0, 0, 0.0)


def test_planted_top_p_before_top_k_is_caught():
    """Filtering by top-p first, then top-k, is a different sampler."""
    logits = [math.log(x) for x in (0.4, 0.35, 0.1, 0.1, 0.05)]
    t, k, p = 1.0, 2, 0.5          # top-k first: 0.53 / 0.47 -> only token 0 reaches 0.5

    def swapped(logits, t, k, p):
        q = brute(logits, t, 0, p)
        live = [i for i in range(len(q)) if q[i] > 0]
        top = sorted(live, key=lambda i: -q[i])[:k]
        tot = sum(q[i] for i in top)
        return [q[i] / tot if i in top else 0.0 for i in range(len(q))]
    got = sampler.probabilities(logits, t, k, p)
    assert got[0] == pytest.approx(1.0) and got[1] == 0
    assert not np.allclose(swapped(logits, t, k, p), got)
