"""One dual-flow decoder layer at one decode step -- test infrastructure only.

What it follows:

* [DFT-pt] "Arquitetura Central": two residual streams share the attention, MLP
  and output matrices; they differ in their token embeddings and a few learned
  coupling vectors. The primary flow writes the persistent KV cache and does
  not depend on the auxiliary flow; the auxiliary flow reads the primary cache,
  never writes it, and never feeds back into the primary flow.
* [DFT-pt] "Mecanismos Chave": coupling vectors a_l, b_l, c_l carry information
  one way, primary to auxiliary, at the query, MLP-intermediate and MLP-output
  levels; the auxiliary query attends the primary keys and values.
* [DFT-pt] "Custos de Inferência vs. Treinamento": at decode both flows read the
  same weights and the same single KV cache.

Layer computed (float64; weights W are [out, in] so ``x W^T``; x1, x2 are the
two flows' residual inputs at this position, the aux one coming from the
aux flow's own embedding):

    q1 = x1 Wq^T   k1 = x1 Wk^T   v1 = x1 Wv^T   q2 = x2 Wq^T     (aux makes no k, v)
    cache slot L_b of sequence b <- bf16(k1), bf16(v1)            (primary only)
    o_f = attention of q^f over the L_b + 1 cached positions     (q^2 = q2 + a * q1)
    h_f = x_f + o_f Wo^T
    z_f = silu(h_f Wg^T) * (h_f Wu^T)        silu(u) = u / (1 + exp(-u))
    z2' = z2 + b * z1
    m1 = z1 Wd^T    m2 = z2' Wd^T    m2' = m2 + c * m1
    out1 = h1 + m1  out2 = h2 + m2'

The coupling formulas for b and c are this library's reading (the pages name
the levels only): additive Hadamard terms, the same form as the query coupling.
No normalisation, no RoPE, no biases.
"""
from typing import Dict

import numpy as np

from .attention import decode_attention
from .formats import f64_to_bf16_bits, to_f64


def linear(x: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """x W^T with W given as bf16 bits of shape [out, in]."""
    return x @ to_f64(w_bits, "bf16").T


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def couple(aux: np.ndarray, vec: np.ndarray, primary: np.ndarray) -> np.ndarray:
    """aux + vec * primary (elementwise; vec broadcast over the batch)."""
    return aux + vec * primary


def append_kv(k_cache, v_cache, block_table, ctx_lens, k_bits, v_bits, block_size: int):
    """Copies of the caches with slot ctx_lens[b] of every sequence set to k_bits/v_bits [B, Hkv, D]."""
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    for b in range(k_bits.shape[0]):
        pos = int(ctx_lens[b])
        blk = int(block_table[b, pos // block_size])
        if blk < 0:
            raise ValueError("no cache block for the appended position")
        slot = pos % block_size
        k_new[blk, :, slot // 16, :, slot % 16, :] = k_bits[b].reshape(k_bits.shape[1], -1, 8)
        v_new[blk, :, slot // 16, :, slot % 16] = v_bits[b]
    return k_new, v_new


def dual_flow_layer(x1, x2, w: Dict[str, np.ndarray], a, b, c, k_cache, v_cache, block_table,
                    ctx_lens, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    scale: float, block_size: int) -> Dict[str, np.ndarray]:
    """All intermediate and final tensors of one layer step (float64; cache slots as bf16 bits)."""
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    bsz = x1.shape[0]
    r = {}
    r["q1"] = linear(x1, w["wq"])
    r["k1"] = linear(x1, w["wk"])
    r["v1"] = linear(x1, w["wv"])
    r["q2"] = linear(x2, w["wq"])
    r["k1_bits"] = f64_to_bf16_bits(r["k1"]).reshape(bsz, num_kv_heads, head_dim)
    r["v1_bits"] = f64_to_bf16_bits(r["v1"]).reshape(bsz, num_kv_heads, head_dim)
    k_new, v_new = append_kv(k_cache, v_cache, block_table, ctx_lens, r["k1_bits"], r["v1_bits"],
                             block_size)
    r["k_cache"], r["v_cache"] = k_new, v_new
    lens = np.asarray(ctx_lens, dtype=np.int64) + 1
    att = decode_attention(r["q1"].reshape(bsz, num_q_heads, head_dim),
                           r["q2"].reshape(bsz, num_q_heads, head_dim),
                           np.asarray(a, dtype=np.float64).reshape(num_q_heads, head_dim),
                           k_new, v_new, block_table, lens, num_kv_heads=num_kv_heads,
                           scale=scale, block_size=block_size, num_flows=2,
                           q_dtype="f64", kv_dtype="bf16")
    r["o1"] = att["o1"].reshape(bsz, -1)
    r["o2"] = att["o2"].reshape(bsz, -1)
    r["h1"] = x1 + linear(r["o1"], w["wo"])
    r["h2"] = x2 + linear(r["o2"], w["wo"])
    r["z1"] = silu(linear(r["h1"], w["wg"])) * linear(r["h1"], w["wu"])
    r["z2"] = silu(linear(r["h2"], w["wg"])) * linear(r["h2"], w["wu"])
    r["z2c"] = couple(r["z2"], np.asarray(b, dtype=np.float64), r["z1"])
    r["m1"] = linear(r["z1"], w["wd"])
    r["m2"] = linear(r["z2c"], w["wd"])
    r["m2c"] = couple(r["m2"], np.asarray(c, dtype=np.float64), r["m1"])
    r["out1"] = r["h1"] + r["m1"]
    r["out2"] = r["h2"] + r["m2c"]
    return r
