"""Mixture of the two flows' next-token distributions -- test infrastructure only.

What it follows: [DFT-pt] "Mecanismos Chave", mixture objective: the final
prediction mixes the primary and auxiliary distributions,

    p_mix = alpha_t * p_primary + (1 - alpha_t) * p_aux,

with alpha_t set from the confidence (collision probability) of the primary
distribution so that the primary keeps at least half of the weight.

The pages give no formula for alpha_t. This library's reading (the plainest
one that meets both stated properties): with the collision probability
c = sum_v p_primary(v)^2, which lies in [1/V, 1],

    alpha_t = (1 + c) / 2,                 so alpha_t in [1/2 + 1/(2V), 1].

A confident primary (c near 1) keeps almost all of the weight; a flat one
keeps just over half.

Decoding the mixture (test-side definitions the kernels must reproduce):

* inverse-CDF sampling with a caller-supplied uniform u in [0, 1): the token
  is the smallest v with sum_{w <= v} p_mix(w) > u * sum_w p_mix(w);
* greedy: the smallest v with the largest p_mix(v).

All in float64 from float32 logits.
"""
from typing import Dict

import numpy as np


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row softmax of [..., V] in float64."""
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def mixture(logits1: np.ndarray, logits2: np.ndarray, u=None) -> Dict[str, np.ndarray]:
    """Mixture of the flows' distributions for a batch of rows.

    logits1, logits2: [B, V] (primary, auxiliary). u: [B] uniforms in [0, 1)
    or None. Returns p1, p2, collision [B], alpha [B], p_mix [B, V],
    greedy [B] and, with u, token [B]."""
    p1 = softmax(logits1)
    p2 = softmax(logits2)
    collision = (p1 * p1).sum(axis=-1)
    alpha = 0.5 * (1.0 + collision)
    p_mix = alpha[:, None] * p1 + (1.0 - alpha[:, None]) * p2
    out = {"p1": p1, "p2": p2, "collision": collision, "alpha": alpha, "p_mix": p_mix,
           "greedy": np.argmax(p_mix, axis=-1).astype(np.int32)}
    if u is not None:
        out["token"] = sample(p_mix, u)
    return out


def sample(p: np.ndarray, u) -> np.ndarray:
    """Inverse-CDF draw per row: the smallest v with cumsum(p)[v] > u * sum(p)."""
    p = np.asarray(p, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    cdf = np.cumsum(p, axis=-1)
    target = u * cdf[:, -1]
    tok = np.empty(p.shape[0], dtype=np.int32)
    for b in range(p.shape[0]):
        above = np.nonzero(cdf[b] > target[b])[0]
        tok[b] = above[0] if above.size else p.shape[1] - 1
    return tok


def cdf_bounds(p: np.ndarray, token: np.ndarray):
    """(sum of p before token, sum up to and including token), normalised by the row total:
    a draw u selected `token` exactly when lo <= u < hi."""
    p = np.asarray(p, dtype=np.float64)
    cdf = np.cumsum(p, axis=-1) / p.sum(axis=-1, keepdims=True)
    rows = np.arange(p.shape[0])
    hi = cdf[rows, token]
    lo = np.where(token > 0, cdf[rows, np.maximum(token - 1, 0)], 0.0)
    return lo, hi
