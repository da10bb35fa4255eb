"""Plain reference of the next-token sampler: temperature, top-k, top-p, sample.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU-baseline
leg, never by the product path.  It shares no code with the GPU kernel.

The steps follow "vLLM 基本原理" (section FlashInfer 采样器 / 工作原理), in its
order: the model's logits are divided by the temperature; top-k keeps the K
most probable tokens; top-p keeps the most probable tokens whose cumulative
probability reaches P; the next token is drawn from what is left, in
proportion to its probability.  The pages ask only that a fast sampler be
statistically equivalent to this; the plain definition is written out here
in float64.

Readings where the pages are silent (listed with the design notes):
* Temperature must be positive (greedy decoding is top_k = 1).
* top_k <= 0 or top_k >= vocabulary size: no top-k filter.  Otherwise a token
  is kept if its logit is at least the K-th largest logit, so tokens tied
  with the K-th are all kept.
* Top-p acts on the probabilities renormalised after top-k: a token is kept
  if the probability mass of the tokens strictly more probable than it is
  below P -- the smallest set of most probable tokens that reaches P, with
  ties at its edge kept.  P must be in (0, 1]; P = 1 keeps everything.
* The draw takes a uniform number u in [0, 1) as input and returns the first
  token, in vocabulary order, whose cumulative probability exceeds u (the
  inverse of the distribution function): a sampler that is deterministic
  given u, so it can be compared draw by draw.
* NaN logits count as -inf; tokens with +inf logits share all the
  probability equally.  A row with no finite logit returns -1.
"""
from __future__ import annotations

import numpy as np


def probabilities(logits, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """Final float64 distribution over the vocabulary (zeros where dropped)."""
    if not temperature > 0:
        raise ValueError("temperature must be positive")
    if not 0 < top_p <= 1:
        raise ValueError("top_p must be in (0, 1]")
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = np.where(np.isnan(z), -np.inf, z)
    v = z.shape[0]
    live = z > -np.inf
    if not live.any():
        return np.zeros(v)
    if np.isposinf(z).any():
        w = np.isposinf(z).astype(np.float64)
    else:
        w = np.where(live, np.exp(z - z[live].max()), 0.0)
    keep = live.copy()
    if 0 < top_k < v:
        kth = np.sort(z)[::-1][top_k - 1]
        keep &= z >= kth
    p = np.where(keep, w, 0.0)
    p = p / p.sum()
    if top_p < 1:
        # mass of the tokens strictly more probable than each token
        order = np.sort(p)[::-1]
        csum = np.concatenate([[0.0], np.cumsum(order)])
        above = csum[np.searchsorted(-order, -p, side="left")]
        keep &= above < top_p
        p = np.where(keep, p, 0.0)
        p = p / p.sum()
    return p


def sample(logits, temperature: float, top_k: int, top_p: float, u: float) -> int:
    """The token the inverse distribution function gives for u in [0, 1)."""
    p = probabilities(logits, temperature, top_k, top_p)
    if not p.any():
        return -1
    c = np.cumsum(p)
    i = int(np.searchsorted(c, u, side="right"))
    kept = np.nonzero(p > 0)[0]
    return int(min(i, kept[-1]))


def sample_batch(logits, temperature, top_k, top_p, u) -> np.ndarray:
    """Row-wise sample over [S, V] logits with per-row parameters."""
    return np.array([sample(logits[s], temperature[s], top_k[s], top_p[s], u[s])
                     for s in range(len(logits))], dtype=np.int64)
