"""Seeded synthetic inputs for dual-flow decode.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds none of the method's arithmetic: it only draws random
numbers, encodes the draws as bf16 bit patterns, and lays them out in the
key/value cache format the library reads. Everything is deterministic in the
seed: every (sequence, kv head, tensor) chunk has its own generator derived
from ``[seed, tag, b, g]``, so any chunk can be regenerated on its own.

Cache layout (one layer), shared by every consumer:

* ``k_cache``: ``[num_blocks, num_kv_heads, block_size // 16, head_dim // 8, 16, 8]``
  -- keys in tiles of 16 positions; inside a tile, groups of 8 dimensions, and
  inside a group the 16 positions' 8 elements each (a tile is one contiguous
  run of 16 * head_dim elements).
* ``v_cache``: ``[num_blocks, num_kv_heads, block_size // 16, head_dim, 16]`` --
  values transposed inside tiles of 16 positions: for each tile and dimension,
  the 16 positions are contiguous.
* ``block_size`` is a multiple of 16 and ``head_dim`` a multiple of 8.
* ``block_table``: int32 ``[batch, max_blocks_per_seq]``; logical block ``j``
  of sequence ``b`` lives in physical block ``block_table[b, j]``; unused
  entries hold -1. A "contiguous" cache is the special case of one block per
  sequence whose size is the capacity.

bf16 tensors are held as ``uint16`` bit patterns; fp32 tensors as ``float32``.
Unused cache slots are filled with NaN so that any read of them shows up.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)

# Tags separating the random streams of different tensors.
_TAG = {"q1": 1, "q2": 2, "a": 3, "k": 4, "v": 5, "peak": 6, "len": 7, "perm": 8,
        "x1": 11, "x2": 12, "wq": 13, "wk": 14, "wv": 15, "wo": 16, "wg": 17,
        "wu": 18, "wd": 19, "b": 20, "c": 21, "l1": 22, "l2": 23, "u": 24, "lpeak": 25, "wlm": 26,
        "h1": 27, "h2": 28, "mh1": 29, "mh2": 30, "mg": 31, "mu": 32, "md": 33, "mr": 34, "mb": 35, "mc": 36,
        "mres1": 37, "mres2": 38, "pq": 39, "pk": 40, "pv": 41, "pq2": 42, "pa": 43, "na": 44, "nm": 45}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return bits.

    Used only to encode random draws; NaN/Inf are never drawn.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tag: str, *idx: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TAG[tag], *[int(i) for i in idx]])


def _normal(seed: int, tag: str, idx: Tuple[int, ...], shape, std: float = 1.0) -> np.ndarray:
    x = _rng(seed, tag, *idx).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


# --------------------------------------------------------------------------
# Attention workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class AttnConfig:
    """One decode-attention workload: shapes, element type, lengths, paging."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # element type of Q1, Q2, K and V: "f32" or "bf16"
    ctx_lens: Optional[Tuple[int, ...]] = None  # explicit per-sequence lengths
    ctx_range: Optional[Tuple[int, int]] = None  # inclusive uniform range when drawn
    block_size: int = 0  # 0: contiguous cache (one block per sequence)
    capacity: int = 0  # contiguous capacity; 0: next power of two >= max length (at least 16)
    shuffle_blocks: bool = False
    peaky_fraction: float = 0.0  # fraction of key rows per (b, kv head) scaled
    peaky_factor: float = 1.0
    q_std: float = 1.0
    kv_std: float = 1.0
    a_std: float = 0.1
    q_dtype: Optional[str] = None  # element type of Q1, Q2 when it differs from the cache's

    @property
    def qtype(self) -> str:
        return self.q_dtype or self.dtype

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "AttnConfig":
        return dataclasses.replace(self, **kw)


# The five decode workloads. C1-C4 are attention-only; C5 is the full layer.
C1 = AttnConfig("c1", batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64, dtype="f32",
                ctx_lens=(512,))
C2 = AttnConfig("c2", batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                ctx_lens=(4096,) * 16)
C3 = AttnConfig("c3", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16",
                ctx_range=(1024, 8192), block_size=16, shuffle_blocks=True)
C4 = AttnConfig("c4", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                ctx_lens=(131072,) * 4, peaky_fraction=0.01, peaky_factor=8.0)
# 16 query heads per kv head (a 128/8-head model): 32 query rows per kv head with both flows
G16 = AttnConfig("g16", batch=8, num_q_heads=128, num_kv_heads=8, head_dim=128, dtype="bf16",
                 ctx_lens=(16384,) * 8)
ATTN_CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "g16": G16}
SEEDS = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5": 1005, "head": 1006, "mix": 1007, "moe": 1008,
         "prefill": 1009, "stack": 1010, "g16": 1011}


def draw_ctx_lens(cfg: AttnConfig, seed: int) -> np.ndarray:
    if cfg.ctx_lens is not None:
        lens = np.asarray(cfg.ctx_lens, dtype=np.int32)
        if lens.shape != (cfg.batch,):
            raise ValueError("ctx_lens must have one entry per sequence")
        return lens
    lo, hi = cfg.ctx_range
    return _rng(seed, "len").integers(lo, hi + 1, size=cfg.batch).astype(np.int32)


@dataclass
class CacheLayout:
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    block_table: np.ndarray  # int32 [batch, max_blocks_per_seq], -1 padded


def plan_cache(batch: int, ctx_lens: np.ndarray, block_size: int, capacity: int,
               shuffle: bool, seed: int, extra_slots: int = 0) -> CacheLayout:
    """Physical block assignment. ``extra_slots`` reserves room past each length."""
    need = ctx_lens.astype(np.int64) + extra_slots
    if block_size == 0:
        cap = capacity or max(16, 1 << int(math.ceil(math.log2(max(int(need.max()), 1)))))
        if need.max() > cap:
            raise ValueError("capacity smaller than a sequence")
        table = np.arange(batch, dtype=np.int32).reshape(batch, 1)
        return CacheLayout(cap, batch, 1, table)
    nblk = (need + block_size - 1) // block_size
    total = int(nblk.sum())
    phys = _rng(seed, "perm").permutation(total).astype(np.int32) if shuffle \
        else np.arange(total, dtype=np.int32)
    mb = int(nblk.max())
    table = np.full((batch, mb), -1, dtype=np.int32)
    pos = 0
    for b in range(batch):
        n = int(nblk[b])
        table[b, :n] = phys[pos:pos + n]
        pos += n
    return CacheLayout(block_size, total, mb, table)


def kv_rows(cfg_seed: int, b: int, g: int, length: int, head_dim: int, dtype: str,
            kv_std: float = 1.0, peaky_fraction: float = 0.0, peaky_factor: float = 1.0):
    """Logical key and value rows of one (sequence, kv head): two [length, head_dim] arrays.

    Returned encoded (bf16 bits or float32)."""
    k = _normal(cfg_seed, "k", (b, g), (length, head_dim), kv_std)
    if peaky_fraction > 0.0:
        n_peak = int(round(peaky_fraction * length))
        rows = _rng(cfg_seed, "peak", b, g).choice(length, size=n_peak, replace=False)
        k[rows] *= np.float32(peaky_factor)
    v = _normal(cfg_seed, "v", (b, g), (length, head_dim), kv_std)
    return _encode(k, dtype), _encode(v, dtype)


def empty_cache(layout: CacheLayout, num_kv_heads: int, head_dim: int, dtype: str):
    bs = layout.block_size
    if bs % 16 or head_dim % 8:
        raise ValueError("block_size must be a multiple of 16 and head_dim of 8")
    shape_k = (layout.num_blocks, num_kv_heads, bs // 16, head_dim // 8, 16, 8)
    shape_v = (layout.num_blocks, num_kv_heads, bs // 16, head_dim, 16)
    if dtype == "bf16":
        return (np.full(shape_k, BF16_NAN_BITS, dtype=np.uint16),
                np.full(shape_v, BF16_NAN_BITS, dtype=np.uint16))
    return (np.full(shape_k, np.nan, dtype=np.float32), np.full(shape_v, np.nan, dtype=np.float32))


def store_rows(k_cache, v_cache, layout: CacheLayout, b: int, g: int, k_rows, v_rows, start: int = 0):
    """Write logical rows [start, start+n) of (b, g) into the paged cache."""
    bs = layout.block_size
    pos = np.arange(start, start + k_rows.shape[0])
    blk = layout.block_table[b, pos // bs].astype(np.int64)
    if np.any(blk < 0):
        raise ValueError("position outside the allocated blocks")
    slot = pos % bs
    n, d = k_rows.shape
    k_cache[blk, g, slot // 16, :, slot % 16, :] = k_rows.reshape(n, d // 8, 8)
    v_cache[blk, g, slot // 16, :, slot % 16] = v_rows


@dataclass
class AttnCase:
    cfg: AttnConfig
    seed: int
    q1: np.ndarray
    q2: np.ndarray
    a: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    ctx_lens: np.ndarray
    block_size: int
    max_blocks_per_seq: int
    extra: Dict[str, np.ndarray] = field(default_factory=dict)

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max())


def make_attn_case(cfg: AttnConfig, seed: int, pad_nan: bool = True) -> AttnCase:
    """All inputs of one decode-attention call for workload ``cfg``."""
    lens = draw_ctx_lens(cfg, seed)
    layout = plan_cache(cfg.batch, lens, cfg.block_size, cfg.capacity, cfg.shuffle_blocks, seed)
    q1 = _encode(_normal(seed, "q1", (), (cfg.batch, cfg.num_q_heads, cfg.head_dim), cfg.q_std), cfg.qtype)
    q2 = _encode(_normal(seed, "q2", (), (cfg.batch, cfg.num_q_heads, cfg.head_dim), cfg.q_std), cfg.qtype)
    a = _normal(seed, "a", (), (cfg.num_q_heads, cfg.head_dim), cfg.a_std)
    k_cache, v_cache = empty_cache(layout, cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
    if not pad_nan:
        k_cache[...] = 0
        v_cache[...] = 0
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            kr, vr = kv_rows(seed, b, g, int(lens[b]), cfg.head_dim, cfg.dtype, cfg.kv_std,
                             cfg.peaky_fraction, cfg.peaky_factor)
            store_rows(k_cache, v_cache, layout, b, g, kr, vr)
    return AttnCase(cfg, seed, q1, q2, a, k_cache, v_cache, layout.block_table, lens,
                    layout.block_size, layout.max_blocks_per_seq)


# --------------------------------------------------------------------------
# Full-layer workload
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerConfig:
    """One dual-flow decoder layer at one decode step."""

    name: str
    batch: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    mlp: int
    ctx: int  # cached positions before this step's append
    block_size: int = 0  # 0: contiguous
    capacity: int = 0
    shuffle_blocks: bool = False
    w_std: float = 0.02
    x_std: float = 1.0
    kv_std: float = 1.0
    coupling_std: float = 0.1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


C5 = LayerConfig("c5", batch=32, hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 mlp=14336, ctx=4096, capacity=8192)


@dataclass
class LayerCase:
    cfg: LayerConfig
    seed: int
    x1: np.ndarray  # float32 [B, hidden], values exactly representable in bf16
    x2: np.ndarray
    w: Dict[str, np.ndarray]  # bf16 bits, [out, in] row-major
    a: np.ndarray  # float32 [Hq * D]
    b: np.ndarray  # float32 [mlp]
    c: np.ndarray  # float32 [hidden]
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    ctx_lens: np.ndarray  # positions cached before the append
    block_size: int
    max_blocks_per_seq: int


def weight_shapes(cfg: LayerConfig) -> Dict[str, Tuple[int, int]]:
    qd, kd = cfg.num_q_heads * cfg.head_dim, cfg.num_kv_heads * cfg.head_dim
    return {"wq": (qd, cfg.hidden), "wk": (kd, cfg.hidden), "wv": (kd, cfg.hidden),
            "wo": (cfg.hidden, qd), "wg": (cfg.mlp, cfg.hidden), "wu": (cfg.mlp, cfg.hidden),
            "wd": (cfg.hidden, cfg.mlp)}


def make_layer_case(cfg: LayerConfig, seed: int, pad_nan: bool = True) -> LayerCase:
    """All inputs of one dual-flow layer step for workload ``cfg``."""
    lens = np.full(cfg.batch, cfg.ctx, dtype=np.int32)
    layout = plan_cache(cfg.batch, lens, cfg.block_size, cfg.capacity, cfg.shuffle_blocks, seed,
                        extra_slots=1)
    x1 = bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, "x1", (), (cfg.batch, cfg.hidden), cfg.x_std)))
    x2 = bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, "x2", (), (cfg.batch, cfg.hidden), cfg.x_std)))
    w = {name: f32_to_bf16_bits(_normal(seed, name, (), shape, cfg.w_std))
         for name, shape in weight_shapes(cfg).items()}
    a = _normal(seed, "a", (), (cfg.num_q_heads * cfg.head_dim,), cfg.coupling_std)
    bvec = _normal(seed, "b", (), (cfg.mlp,), cfg.coupling_std)
    cvec = _normal(seed, "c", (), (cfg.hidden,), cfg.coupling_std)
    k_cache, v_cache = empty_cache(layout, cfg.num_kv_heads, cfg.head_dim, "bf16")
    if not pad_nan:
        k_cache[...] = 0
        v_cache[...] = 0
    for bi in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            kr, vr = kv_rows(seed, bi, g, cfg.ctx, cfg.head_dim, "bf16", cfg.kv_std)
            store_rows(k_cache, v_cache, layout, bi, g, kr, vr)
    return LayerCase(cfg, seed, x1, x2, w, a, bvec, cvec, k_cache, v_cache, layout.block_table,
                     lens, layout.block_size, layout.max_blocks_per_seq)


def permute_blocks(k_cache, v_cache, block_table, seed: int):
    """Same logical cache under a different physical block order (a layout-only change)."""
    nb = k_cache.shape[0]
    perm = np.random.default_rng([int(seed), 99]).permutation(nb)  # new position of old block i
    k2 = np.empty_like(k_cache)
    v2 = np.empty_like(v_cache)
    k2[perm] = k_cache
    v2[perm] = v_cache
    t2 = np.where(block_table >= 0, perm[np.maximum(block_table, 0)], -1).astype(np.int32)
    return k2, v2, t2


# --------------------------------------------------------------------------
# Output-head workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class MixConfig:
    """Next-token logits of both flows for a batch of sequences.

    Logits are normal draws with standard deviation ``std``; in a fraction
    ``peak_rows`` of the sequences, ``peak_tokens`` random tokens of each
    flow's row get ``peak_boost`` added (a confident distribution)."""

    name: str
    batch: int
    vocab: int
    std: float = 2.0
    peak_rows: float = 0.5
    peak_tokens: int = 4
    peak_boost: float = 12.0

    def replace(self, **kw) -> "MixConfig":
        return dataclasses.replace(self, **kw)


def make_mixture_case(cfg: MixConfig, seed: int):
    """(logits1, logits2, u): float32 [batch, vocab] twice and float32 [batch] in [0, 1)."""
    l1 = _normal(seed, "l1", (), (cfg.batch, cfg.vocab), cfg.std)
    l2 = _normal(seed, "l2", (), (cfg.batch, cfg.vocab), cfg.std)
    rng = _rng(seed, "lpeak")
    for b in range(cfg.batch):
        if rng.random() < cfg.peak_rows:
            for row in (l1, l2):
                row[b, rng.choice(cfg.vocab, size=min(cfg.peak_tokens, cfg.vocab), replace=False)] += \
                    np.float32(cfg.peak_boost)
    u = _rng(seed, "u").random(cfg.batch, dtype=np.float32)
    return l1, l2, u


@dataclass(frozen=True)
class HeadConfig:
    """Shared output head: both flows' final hidden states times one vocabulary matrix."""

    name: str
    batch: int
    hidden: int
    vocab: int
    x_std: float = 1.0
    w_std: float = 0.02

    def replace(self, **kw) -> "HeadConfig":
        return dataclasses.replace(self, **kw)


# The output head after the C5 layer: batch 32, hidden 4096, weights ~ N(0, 0.02). The pages
# name no vocabulary; 32000 tokens is the size used with hidden 4096 by the common 7B models.
HEAD = HeadConfig("head", batch=32, hidden=4096, vocab=32000)
MIX = MixConfig("mix", batch=32, vocab=32000)


def make_head_case(cfg: HeadConfig, seed: int):
    """(h1, h2, w_bits, u): hidden states float32 [batch, hidden] (exact bf16 values), the
    vocabulary matrix as bf16 bits [vocab, hidden] (row-major), uniforms float32 [batch]."""
    h1 = bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, "h1", (), (cfg.batch, cfg.hidden), cfg.x_std)))
    h2 = bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, "h2", (), (cfg.batch, cfg.hidden), cfg.x_std)))
    w = f32_to_bf16_bits(_normal(seed, "wlm", (), (cfg.vocab, cfg.hidden), cfg.w_std))
    u = _rng(seed, "u").random(cfg.batch, dtype=np.float32)
    return h1, h2, w, u


# --------------------------------------------------------------------------
# Mixture-of-experts workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class MoeConfig:
    """A SwiGLU mixture-of-experts FFN at one decode step: `experts` experts of width `mlp`, a
    shared router, primary fan-out k1 and auxiliary fan-out k2 (k1 <= k2)."""

    name: str
    batch: int
    hidden: int
    mlp: int
    experts: int
    k1: int
    k2: int
    w_std: float = 0.02
    x_std: float = 1.0
    coupling_std: float = 0.1

    def replace(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


# The MoE FFN after the C5 attention block: batch 32, hidden 4096, weights ~ N(0, 0.02); 64
# experts of width 1024 with the primary taking its top 4 and the auxiliary flow the top 8 of the
# primary's ranking. The pages name no expert configuration.
MOE = MoeConfig("moe", batch=32, hidden=4096, mlp=1024, experts=64, k1=4, k2=8)


@dataclass
class MoeCase:
    cfg: MoeConfig
    h1: np.ndarray    # float32 [B, hidden], exact bf16 values (the FFN inputs)
    h2: np.ndarray
    res1: np.ndarray  # float32 [B, hidden] (residual stream added to the FFN output)
    res2: np.ndarray
    wg: np.ndarray    # bf16 bits [E, mlp, hidden]
    wu: np.ndarray    # bf16 bits [E, mlp, hidden]
    wd: np.ndarray    # bf16 bits [E, hidden, mlp]
    wr: np.ndarray    # bf16 bits [E, hidden] router
    b: np.ndarray     # float32 [mlp]
    c: np.ndarray     # float32 [hidden]


def make_moe_case(cfg: MoeConfig, seed: int) -> MoeCase:
    """All inputs of one MoE FFN step (router logits are h_f Wr^T, computed by the consumer)."""
    def acts(tag):
        return bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, tag, (), (cfg.batch, cfg.hidden), cfg.x_std)))
    wg = np.stack([f32_to_bf16_bits(_normal(seed, "mg", (e,), (cfg.mlp, cfg.hidden), cfg.w_std))
                   for e in range(cfg.experts)])
    wu = np.stack([f32_to_bf16_bits(_normal(seed, "mu", (e,), (cfg.mlp, cfg.hidden), cfg.w_std))
                   for e in range(cfg.experts)])
    wd = np.stack([f32_to_bf16_bits(_normal(seed, "md", (e,), (cfg.hidden, cfg.mlp), cfg.w_std))
                   for e in range(cfg.experts)])
    wr = f32_to_bf16_bits(_normal(seed, "mr", (), (cfg.experts, cfg.hidden), cfg.w_std))
    return MoeCase(cfg, acts("mh1"), acts("mh2"), _normal(seed, "mres1", (), (cfg.batch, cfg.hidden)),
                   _normal(seed, "mres2", (), (cfg.batch, cfg.hidden)), wg, wu, wd, wr,
                   _normal(seed, "mb", (), (cfg.mlp,), cfg.coupling_std),
                   _normal(seed, "mc", (), (cfg.hidden,), cfg.coupling_std))


# --------------------------------------------------------------------------
# Prefill workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefillConfig:
    """Prompts processed by the primary flow (causal self-attention), written to a paged cache."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lens: Tuple[int, ...]     # prompt lengths
    block_size: int = 16
    shuffle_blocks: bool = True
    extra_slots: int = 16     # cache room past each prompt (the decode steps that follow)
    std: float = 1.0
    a_std: float = 0.1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


# Prompts of 4096 tokens, batch 4, 32/8 heads of 128 (the decode workloads' attention shape).
PREFILL = PrefillConfig("prefill", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, lens=(4096,) * 4)


@dataclass
class PrefillCase:
    cfg: PrefillConfig
    q: np.ndarray        # bf16 bits [B, Lmax, Hq, D]: the primary's queries over the prompt
    k: np.ndarray        # bf16 bits [B, Lmax, Hkv, D]
    v: np.ndarray
    lens: np.ndarray     # int32 [B]
    q2: np.ndarray       # bf16 bits [B, Hq, D]: the auxiliary query at the last prompt position
    a: np.ndarray        # float32 [Hq * D]
    k_cache: np.ndarray  # empty paged cache (NaN) that the prefill fills
    v_cache: np.ndarray
    block_table: np.ndarray
    block_size: int
    max_blocks_per_seq: int


def make_prefill_case(cfg: PrefillConfig, seed: int) -> PrefillCase:
    lens = np.asarray(cfg.lens, dtype=np.int32)
    if lens.shape != (cfg.batch,):
        raise ValueError("one length per prompt")
    lmax = int(lens.max())
    layout = plan_cache(cfg.batch, lens, cfg.block_size, 0, cfg.shuffle_blocks, seed, extra_slots=cfg.extra_slots)
    q = f32_to_bf16_bits(_normal(seed, "pq", (), (cfg.batch, lmax, cfg.num_q_heads, cfg.head_dim), cfg.std))
    k = f32_to_bf16_bits(_normal(seed, "pk", (), (cfg.batch, lmax, cfg.num_kv_heads, cfg.head_dim), cfg.std))
    v = f32_to_bf16_bits(_normal(seed, "pv", (), (cfg.batch, lmax, cfg.num_kv_heads, cfg.head_dim), cfg.std))
    q2 = f32_to_bf16_bits(_normal(seed, "pq2", (), (cfg.batch, cfg.num_q_heads, cfg.head_dim), cfg.std))
    a = _normal(seed, "pa", (), (cfg.num_q_heads * cfg.head_dim,), cfg.a_std)
    for b in range(cfg.batch):  # positions past a prompt are NaN: any read of them shows up
        for x in (q, k, v):
            x[b, lens[b]:] = BF16_NAN_BITS
    k_cache, v_cache = empty_cache(layout, cfg.num_kv_heads, cfg.head_dim, "bf16")
    return PrefillCase(cfg, q, k, v, lens, q2, a, k_cache, v_cache, layout.block_table, layout.block_size,
                       layout.max_blocks_per_seq)


# --------------------------------------------------------------------------
# Layer stacks (one decode step through several layers)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class StackConfig:
    """`layers` dual-flow layers of shape `layer`, optional pre-norm RMSNorm and rotary embeddings."""

    name: str
    layer: LayerConfig
    layers: int
    rope: str = "half"        # "none", "half" or "interleaved"
    rms: bool = True
    eps: float = 1e-5
    norm_std: float = 0.1     # RMSNorm weights ~ 1 + N(0, norm_std)
    rope_base: float = 10000.0

    def replace(self, **kw) -> "StackConfig":
        return dataclasses.replace(self, **kw)


# Four C5-shaped layers (batch 32, hidden 4096, 32/8 heads of 128, SwiGLU 14336, 4096 cached positions
# per layer) with RMSNorm and rotate-half rotary embeddings.
STACK = StackConfig("stack", C5, layers=4)


def rope_tables(max_pos: int, head_dim: int, base: float = 10000.0):
    """The conventional rotary angle tables (model configuration, like the weights): angle
    p * base^(-2i / head_dim) for position p and pair i; float32 cos, sin [max_pos, head_dim / 2]."""
    inv = np.power(float(base), -np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclass
class StackCase:
    cfg: StackConfig
    x1: np.ndarray
    x2: np.ndarray
    layers: list           # per layer: dict of wq, wk, wv, wo, wg, wu, wd (bf16 bits), a, b, c, n_attn, n_mlp
    k_caches: list
    v_caches: list
    block_table: np.ndarray
    ctx_lens: np.ndarray
    block_size: int
    max_blocks_per_seq: int
    cos: np.ndarray        # float32 [max_pos, D/2]
    sin: np.ndarray


def make_stack_case(cfg: StackConfig, seed: int, pad_nan: bool = True) -> StackCase:
    """All layers share the cache layout, positions and inputs of make_layer_case(cfg.layer, seed); layer
    l draws its weights, couplings, norms and cached keys/values from seed + 7919 * l (so layer 0 is
    exactly that layer case)."""
    lc = cfg.layer
    lens = np.full(lc.batch, lc.ctx, dtype=np.int32)
    layout = plan_cache(lc.batch, lens, lc.block_size, lc.capacity, lc.shuffle_blocks, seed, extra_slots=1)
    x1 = bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, "x1", (), (lc.batch, lc.hidden), lc.x_std)))
    x2 = bf16_bits_to_f32(f32_to_bf16_bits(_normal(seed, "x2", (), (lc.batch, lc.hidden), lc.x_std)))
    layers, kcs, vcs = [], [], []
    for li in range(cfg.layers):
        sl = seed + 7919 * li
        w = {name: f32_to_bf16_bits(_normal(sl, name, (), shape, lc.w_std)) for name, shape in weight_shapes(lc).items()}
        w.update(a=_normal(sl, "a", (), (lc.num_q_heads * lc.head_dim,), lc.coupling_std),
                 b=_normal(sl, "b", (), (lc.mlp,), lc.coupling_std),
                 c=_normal(sl, "c", (), (lc.hidden,), lc.coupling_std),
                 n_attn=1.0 + _normal(sl, "na", (), (lc.hidden,), cfg.norm_std),
                 n_mlp=1.0 + _normal(sl, "nm", (), (lc.hidden,), cfg.norm_std))
        k_cache, v_cache = empty_cache(layout, lc.num_kv_heads, lc.head_dim, "bf16")
        if not pad_nan:
            k_cache[...] = 0
            v_cache[...] = 0
        for bi in range(lc.batch):
            for g in range(lc.num_kv_heads):
                kr, vr = kv_rows(sl, bi, g, lc.ctx, lc.head_dim, "bf16", lc.kv_std)
                store_rows(k_cache, v_cache, layout, bi, g, kr, vr)
        layers.append(w)
        kcs.append(k_cache)
        vcs.append(v_cache)
    max_pos = layout.max_blocks_per_seq * layout.block_size
    cos, sin = rope_tables(max_pos, lc.head_dim, cfg.rope_base)
    return StackCase(cfg, x1, x2, layers, kcs, vcs, layout.block_table, lens, layout.block_size,
                     layout.max_blocks_per_seq, cos, sin)
