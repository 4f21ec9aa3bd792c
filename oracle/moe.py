"""Mixture-of-experts FFN with router replay, one decode step -- test infrastructure only.

What it follows:

* [DFT-pt] "Mecanismos Chave", router replay: in a mixture-of-experts layer the
  auxiliary flow reuses the experts the primary router selected, and combines
  them with mixing weights of its own.
* [DFT-pt] "Contribuições Principais" (phase-specific MoE allocation) and
  "Significância e Alegações": the primary and auxiliary expert fan-outs are
  set independently (prefill cost follows the primary's experts, decode cost
  the sum of both); [DFT-de] illustrates it as reading with 5 experts and
  writing with 10 or 15.
* [DFT-pt] "Mecanismos Chave", lightweight coupling: b at the MLP intermediate,
  c at the MLP output, primary to auxiliary only (as in the dense layer).

This library's reading (the pages give no formulas). With router logits
r_f = h_f Wr^T over E experts (both flows through the shared router), and
fan-outs k1 <= k2 <= E:

    ranking   experts by r1 descending, ties to the smaller index
    S1, S2    the first k1 and the first k2 experts of that ranking
              (the auxiliary flow replays the primary router: S1 is a prefix of S2)
    g1, g2    softmax of r1 over S1, softmax of r2 over S2 (own mixing weights)
    z_f,e     silu(h_f Wg_e^T) * (h_f Wu_e^T)             (SwiGLU expert e)
    z2,e'     z2,e + b * z1,e for e in S1, else z2,e       (b where the primary ran e)
    m1        sum_{e in S1} g1(e) z1,e Wd_e^T
    m2        sum_{e in S2} g2(e) z2,e' Wd_e^T
    out1      res1 + m1
    out2      res2 + m2 + c * m1

Weights are bf16 bit patterns, [E, out, in] per matrix; everything else float64.
"""
from typing import Dict

import numpy as np

from .formats import to_f64
from .layer import silu


def route(r1: np.ndarray, r2: np.ndarray, k1: int, k2: int) -> Dict[str, np.ndarray]:
    """Selection and mixing weights for a batch: r1, r2 [B, E] router logits.

    Returns sel [B, k2] (experts in ranking order; the first k1 are S1), g1 [B, k1], g2 [B, k2]."""
    r1 = np.asarray(r1, dtype=np.float64)
    r2 = np.asarray(r2, dtype=np.float64)
    if not 1 <= k1 <= k2 <= r1.shape[1]:
        raise ValueError("need 1 <= k1 <= k2 <= number of experts")
    # a stable sort of -r1 keeps equal logits in index order
    sel = np.argsort(-r1, axis=-1, kind="stable")[:, :k2]
    rows = np.arange(r1.shape[0])[:, None]
    g1 = _softmax(r1[rows, sel[:, :k1]])
    g2 = _softmax(r2[rows, sel])
    return {"sel": sel.astype(np.int32), "g1": g1, "g2": g2}


def _softmax(x: np.ndarray) -> np.ndarray:
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def expert(h: np.ndarray, wg_bits: np.ndarray, wu_bits: np.ndarray) -> np.ndarray:
    """SwiGLU intermediate of one expert: silu(h Wg^T) * (h Wu^T)."""
    return silu(h @ to_f64(wg_bits, "bf16").T) * (h @ to_f64(wu_bits, "bf16").T)


def moe_ffn(h1, h2, res1, res2, wg, wu, wd, b, c, sel, g1, g2) -> Dict[str, np.ndarray]:
    """Both flows' outputs for a batch, given the routing of route().

    h1, h2, res1, res2: [B, hidden]; wg, wu: bf16 bits [E, mlp, hidden]; wd: [E, hidden, mlp];
    b: [mlp] or None; c: [hidden] or None. Returns m1, m2 (the MoE outputs before the
    residual, m2 without the c term), out1, out2."""
    h1 = np.asarray(h1, dtype=np.float64)
    h2 = np.asarray(h2, dtype=np.float64)
    bsz, hidden = h1.shape
    k1, k2 = g1.shape[1], g2.shape[1]
    m1 = np.zeros((bsz, hidden))
    m2 = np.zeros((bsz, hidden))
    bv = None if b is None else np.asarray(b, dtype=np.float64)
    for s in range(bsz):
        for slot in range(k2):
            e = int(sel[s, slot])
            wd_e = to_f64(wd[e], "bf16")
            z2 = expert(h2[s:s + 1], wg[e], wu[e])
            if slot < k1:  # e is in S1: the primary runs it, and b couples it into the aux flow
                z1 = expert(h1[s:s + 1], wg[e], wu[e])
                m1[s] += g1[s, slot] * (z1 @ wd_e.T)[0]
                if bv is not None:
                    z2 = z2 + bv * z1
            m2[s] += g2[s, slot] * (z2 @ wd_e.T)[0]
    out1 = np.asarray(res1, dtype=np.float64) + m1
    out2 = np.asarray(res2, dtype=np.float64) + m2
    if c is not None:
        out2 = out2 + np.asarray(c, dtype=np.float64) * m1
    return {"m1": m1, "m2": m2, "out1": out1, "out2": out2}
