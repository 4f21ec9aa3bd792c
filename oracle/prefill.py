"""Primary-only prefill of a prompt, and the auxiliary flow's first step -- test infrastructure only.

What it follows:

* [DFT-pt] "Custos de Inferência vs. Treinamento": prefill costs nothing extra
  over a standard Transformer, the auxiliary flow being skipped there;
  "Arquitetura Central": only the primary flow writes the KV cache.
* [DFT-de] (second and third paragraphs): the primary lane reads the whole
  prompt like a standard model and builds the key/value cache; the auxiliary
  lane skips the reading phase and starts at the last prompt position, where
  it looks at the primary's cache.

Computed (float64; inputs bf16 bit patterns). For every prompt b of length
L_b, query head h, position t < L_b, with kv head g = h // (Hq / Hkv):

    O[b, t, h] = sum_{u <= t} softmax_u(scale * <Q[b, t, h], K[b, u, g]>) V[b, u, g]

(causal self-attention of the primary flow), and the cache holds K[b, u, g],
V[b, u, g] at positions u < L_b of sequence b. The auxiliary flow's first
step is a decode step at position L_b - 1 over the L_b cached positions
(oracle.attention.decode_attention with ctx_lens = L_b).
"""
from typing import Dict

import numpy as np

from .formats import to_f64


def causal_attention(q_bits, k_bits, v_bits, lens, *, num_kv_heads: int, scale: float) -> np.ndarray:
    """q [B, Lmax, Hq, D], k, v [B, Lmax, Hkv, D] (bf16 bits); lens [B]. Returns O [B, Lmax, Hq, D]
    (float64; rows at t >= L_b are zero)."""
    q = to_f64(q_bits, "bf16")
    k = to_f64(k_bits, "bf16")
    v = to_f64(v_bits, "bf16")
    bsz, lmax, hq, d = q.shape
    group = hq // num_kv_heads
    out = np.zeros((bsz, lmax, hq, d))
    for b in range(bsz):
        n = int(lens[b])
        if n == 0:
            continue
        mask = np.tril(np.ones((n, n), dtype=bool))  # row t sees u <= t
        for h in range(hq):
            g = h // group
            s = scale * (q[b, :n, h] @ k[b, :n, g].T)
            s = np.where(mask, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            out[b, :n, h] = w @ v[b, :n, g]
    return out


def cache_after_prefill(k_cache, v_cache, block_table, k_bits, v_bits, lens, block_size: int) -> Dict[str, np.ndarray]:
    """Copies of the caches with positions [0, L_b) of every sequence b set to the prompt's keys and
    values (cache layouts of workloads: k [blocks, Hkv, bs/16, D/8, 16, 8], v [blocks, Hkv, bs/16, D, 16])."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    hkv, d = k_bits.shape[2], k_bits.shape[3]
    for b in range(k_bits.shape[0]):
        for t in range(int(lens[b])):
            blk = int(block_table[b, t // block_size])
            slot = t % block_size
            kc[blk, :, slot // 16, :, slot % 16, :] = k_bits[b, t].reshape(hkv, d // 8, 8)
            vc[blk, :, slot // 16, :, slot % 16] = v_bits[b, t]
    return {"k_cache": kc, "v_cache": vc}
