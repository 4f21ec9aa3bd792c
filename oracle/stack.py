"""A stack of dual-flow decoder layers at one decode step, with RMSNorm and rotary
position embeddings -- test infrastructure only.

What it follows: the layer of oracle/layer.py ([DFT-pt] "Arquitetura Central",
"Mecanismos Chave"), repeated over the layers of a model, each flow's output
feeding the next layer. The pages name no normalisation and no position
encoding; this library offers the LLaMA-like choices as options:

* pre-norm RMSNorm before the attention block and before the MLP block, one
  weight vector per block and layer, shared by both flows (the flows share
  every weight of a layer):   RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w;
* rotary embeddings of both flows' queries and of the primary's key at the
  new position L = ctx_lens[b], applied after the projections and before the
  query coupling and the cache append, as rotations of dimension pairs of
  each head by the angle table (cos, sin)[L][i]:
    "half"        pairs (i, i + D/2)      (rotate-half form)
    "interleaved" pairs (2i, 2i + 1)
  (x, y) -> (x cos - y sin, x sin + y cos).

Per layer (x1, x2 its inputs):

    a_f = RMSNorm(x_f; wn_attn)                    (or x_f)
    q_f = rope(a_f Wq^T),  k1 = rope(a_1 Wk^T),  v1 = a_1 Wv^T
    cache slot L <- bf16(k1), bf16(v1)            (primary only)
    o_f = attention over [0, L] (q2 coupled: rope(q2) + a * rope(q1))
    h_f = x_f + o_f Wo^T
    m_f = RMSNorm(h_f; wn_mlp)                     (or h_f)
    z_f = silu(m_f Wg^T) * (m_f Wu^T),  z2' = z2 + b * z1
    out_1 = h_1 + z_1 Wd^T,  out_2 = h_2 + z2' Wd^T + c * (z_1 Wd^T)
"""
from typing import Dict, List, Optional

import numpy as np

from .attention import decode_attention
from .formats import f64_to_bf16_bits
from .layer import append_kv, couple, linear, silu


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def rope(x: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray, head_dim: int, style: str) -> np.ndarray:
    """x [B, H*D] rotated at positions pos [B] with tables cos, sin [max_pos, D/2]."""
    if style == "none":
        return np.asarray(x, dtype=np.float64)
    bsz = x.shape[0]
    y = np.asarray(x, dtype=np.float64).reshape(bsz, -1, head_dim).copy()
    c = np.asarray(cos, dtype=np.float64)[pos][:, None, :]  # [B, 1, D/2]
    s = np.asarray(sin, dtype=np.float64)[pos][:, None, :]
    if style == "half":
        a, b = y[..., :head_dim // 2].copy(), y[..., head_dim // 2:].copy()
        y[..., :head_dim // 2] = a * c - b * s
        y[..., head_dim // 2:] = a * s + b * c
    elif style == "interleaved":
        a, b = y[..., 0::2].copy(), y[..., 1::2].copy()
        y[..., 0::2] = a * c - b * s
        y[..., 1::2] = a * s + b * c
    else:
        raise ValueError(style)
    return y.reshape(bsz, -1)


def rope_tables(max_pos: int, head_dim: int, base: float = 10000.0):
    """Standard angle tables: theta(p, i) = p * base^(-2i/D). Returns float64 cos, sin [max_pos, D/2]."""
    inv = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def stack_step(x1, x2, layers: List[Dict[str, np.ndarray]], k_caches, v_caches, block_table, ctx_lens, *,
               num_q_heads: int, num_kv_heads: int, head_dim: int, scale: float, block_size: int,
               rope_style: str = "none", cos: Optional[np.ndarray] = None, sin: Optional[np.ndarray] = None,
               rms: bool = False, eps: float = 1e-5) -> Dict[str, object]:
    """All layers' outputs and caches. layers[l] holds wq, wk, wv, wo, wg, wu, wd (bf16 bits), a, b, c
    and, with rms, n_attn, n_mlp."""
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    bsz = x1.shape[0]
    pos = np.asarray(ctx_lens, dtype=np.int64)
    outs, caches = [], []
    for li, w in enumerate(layers):
        a1 = rms_norm(x1, w["n_attn"], eps) if rms else x1
        a2 = rms_norm(x2, w["n_attn"], eps) if rms else x2
        q1 = rope(linear(a1, w["wq"]), pos, cos, sin, head_dim, rope_style)
        q2 = rope(linear(a2, w["wq"]), pos, cos, sin, head_dim, rope_style)
        k1 = rope(linear(a1, w["wk"]), pos, cos, sin, head_dim, rope_style)
        v1 = linear(a1, w["wv"])
        kb = f64_to_bf16_bits(k1).reshape(bsz, num_kv_heads, head_dim)
        vb = f64_to_bf16_bits(v1).reshape(bsz, num_kv_heads, head_dim)
        kc, vc = append_kv(k_caches[li], v_caches[li], block_table, ctx_lens, kb, vb, block_size)
        att = decode_attention(q1.reshape(bsz, num_q_heads, head_dim), q2.reshape(bsz, num_q_heads, head_dim),
                               np.asarray(w["a"], dtype=np.float64).reshape(num_q_heads, head_dim), kc, vc,
                               block_table, pos + 1, num_kv_heads=num_kv_heads, scale=scale,
                               block_size=block_size, num_flows=2, q_dtype="f64", kv_dtype="bf16")
        h1 = x1 + linear(att["o1"].reshape(bsz, -1), w["wo"])
        h2 = x2 + linear(att["o2"].reshape(bsz, -1), w["wo"])
        m1 = rms_norm(h1, w["n_mlp"], eps) if rms else h1
        m2 = rms_norm(h2, w["n_mlp"], eps) if rms else h2
        z1 = silu(linear(m1, w["wg"])) * linear(m1, w["wu"])
        z2 = couple(silu(linear(m2, w["wg"])) * linear(m2, w["wu"]), np.asarray(w["b"], dtype=np.float64), z1)
        d1 = linear(z1, w["wd"])
        x1 = h1 + d1
        x2 = h2 + couple(linear(z2, w["wd"]), np.asarray(w["c"], dtype=np.float64), d1)
        outs.append((x1, x2))
        caches.append((kc, vc))
    return {"out1": x1, "out2": x2, "layers": outs, "caches": caches}
