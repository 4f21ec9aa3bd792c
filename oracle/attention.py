"""Exact softmax attention of both flows over the primary KV cache -- test infrastructure only.

What it follows: [DFT-pt] section "Mecanismos Chave", asymmetric shared-KV
attention: the primary query attends the primary keys and values causally; the
auxiliary flow makes its own query, couples it to the primary query through a
learned vector a_l, and attends the same primary keys and values, never writing
its own. [DFT-pt] "Arquitetura Central": the auxiliary flow reads the primary
cache but never writes it.

Definition computed (float64, no online softmax, no splits), for sequence b,
query head h and flow f in {1, 2}, with g the kv head of h and L_b = ctx_lens[b]:

    q^1 = Q1[b, h]                      q^2 = Q2[b, h] + a[h] * Q1[b, h]
    s_t = scale * <q^f, K_t>            for cached positions t in [0, L_b)
    w_t = exp(s_t - max s) / sum_u exp(s_u - max s)
    O_f[b, h] = sum_t w_t V_t

Decode attends every cached position of the sequence (the new token is the
last one), so no causal mask is needed beyond the length. Cache layout: keys
[num_blocks, Hkv, block/16, D/8, 16, 8] (tiles of 16 positions, inside a tile
8-dimension groups of the 16 positions); values [num_blocks, Hkv, block/16, D,
16] (transposed inside tiles of 16 positions); position t of sequence b is in
block table[b, t // block], slot t % block.
"""
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

from .formats import to_f64


def kv_head_of(h: int, group: int) -> int:
    """Query head h reads kv head h // group (consecutive query heads share a kv head)."""
    return h // group


def coupled_query(q1: np.ndarray, q2: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Auxiliary query after coupling to the primary query: q2 + a * q1 (elementwise)."""
    return q2 + a * q1


def block_rows(table_row: np.ndarray, length: int, block_size: int) -> np.ndarray:
    """Physical block of each of the first ``length`` positions' blocks."""
    nblk = -(-length // block_size)
    blocks = np.asarray(table_row[:nblk], dtype=np.int64)
    if blocks.shape[0] != nblk or np.any(blocks < 0):
        raise ValueError("block table does not cover the context length")
    return blocks


def gather_keys(k_cache, table_row, length: int, g: int, block_size: int, dtype: str) -> np.ndarray:
    """Keys of positions [0, length) of one sequence and kv head, as float64 [length, D]."""
    blocks = block_rows(table_row, length, block_size)
    k = np.swapaxes(k_cache[blocks, g], 2, 3)  # [nblk, block/16, D/8, 16, 8] -> [nblk, block/16, 16, D/8, 8]
    return to_f64(k.reshape(-1, k.shape[3] * k.shape[4])[:length], dtype)


def gather_values(v_cache, table_row, length: int, g: int, block_size: int, dtype: str) -> np.ndarray:
    """Values of positions [0, length) of one sequence and kv head, as float64 [length, D]."""
    blocks = block_rows(table_row, length, block_size)
    v = np.swapaxes(v_cache[blocks, g], 2, 3)  # [nblk, block/16, D, 16] -> [nblk, block/16, 16, D]
    return to_f64(v.reshape(-1, v.shape[-1])[:length], dtype)


def softmax_weights(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum exp(s - max s) over the last axis."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of query rows q [R, D] over keys/values [L, D]."""
    w = softmax_weights((q @ keys.T) * scale)
    return w @ values, w


def decode_attention(q1, q2, a, k_cache, v_cache, block_table, ctx_lens, *,
                     num_kv_heads: int, scale: float, block_size: int, num_flows: int = 2,
                     q_dtype: str = "bf16", kv_dtype: str = "bf16",
                     pairs: Optional[Iterable[Tuple[int, int]]] = None,
                     return_weights: bool = False) -> Dict[str, object]:
    """Both flows' attention outputs for every (b, h), or for the (b, kv head) ``pairs`` given.

    Returns {"o1": [B, Hq, D] float64, "o2": ... (num_flows == 2)}; rows outside
    ``pairs`` are NaN. With ``return_weights`` also {"w": {(b, h, f): weights}}.
    """
    q1 = to_f64(q1, q_dtype)
    batch, hq, d = q1.shape
    group = hq // num_kv_heads
    if group * num_kv_heads != hq:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if num_flows not in (1, 2):
        raise ValueError("num_flows is 1 or 2")
    if num_flows == 2:
        q2 = to_f64(q2, q_dtype)
        a = np.asarray(a, dtype=np.float64).reshape(hq, d)
    wanted = None if pairs is None else set((int(b), int(g)) for b, g in pairs)
    out = {"o1": np.full((batch, hq, d), np.nan)}
    if num_flows == 2:
        out["o2"] = np.full((batch, hq, d), np.nan)
    weights = {}
    heads_of = {}
    for h in range(hq):
        heads_of.setdefault(kv_head_of(h, group), []).append(h)
    for b in range(batch):
        length = int(ctx_lens[b])
        if length < 1:
            raise ValueError("a context holds at least one position")
        for g in sorted(heads_of):
            if wanted is not None and (b, g) not in wanted:
                continue
            keys = gather_keys(k_cache, block_table[b], length, g, block_size, kv_dtype)
            values = gather_values(v_cache, block_table[b], length, g, block_size, kv_dtype)
            for h in heads_of[g]:
                rows = [q1[b, h]]
                if num_flows == 2:
                    rows.append(coupled_query(q1[b, h], q2[b, h], a[h]))
                o, w = attend(np.stack(rows), keys, values, scale)
                for f in range(num_flows):
                    out[f"o{f + 1}"][b, h] = o[f]
                    if return_weights:
                        weights[(b, h, f + 1)] = w[f]
    if return_weights:
        out["w"] = weights
    return out
