"""Pins of the attention oracle: checks against facts other than the oracle itself.

Each pin raises AssertionError when the oracle disagrees with:
brute force (independent scalar code), a library routine (torch's
scaled_dot_product_attention in float64), closed forms (one position, zero
keys, two keys, a dominant key), or invariants (aux == primary special case,
weights summing to one, physical block order, shift of every key by one
vector). ``ALL_PINS`` is the battery; the mutation tests plant mistakes in the
oracle and require the battery to fail.
"""
import math

import numpy as np
import torch

import workloads as W
from oracle import attention as A
from oracle import brute as BR

TINY = [
    # (config, seed): GQA paged + shuffled bf16 with ragged lengths; MHA contiguous f32
    (W.AttnConfig("tiny_gqa", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="bf16",
                  ctx_lens=(5, 50), block_size=16, shuffle_blocks=True), 11),
    (W.AttnConfig("tiny_mha", batch=1, num_q_heads=2, num_kv_heads=2, head_dim=16, dtype="f32",
                  ctx_lens=(9,)), 12),
    (W.AttnConfig("tiny_g4", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=8, dtype="bf16",
                  ctx_lens=(1, 35), block_size=16, shuffle_blocks=True, peaky_fraction=0.2,
                  peaky_factor=8.0), 13),
]


def run_oracle(case, **kw):
    cfg = case.cfg
    args = dict(num_kv_heads=cfg.num_kv_heads, scale=cfg.scale, block_size=case.block_size,
                num_flows=2, q_dtype=cfg.dtype, kv_dtype=cfg.dtype)
    args.update(kw)
    return A.decode_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache,
                              case.block_table, case.ctx_lens, **args)


def pin_brute_force():
    for cfg, seed in TINY:
        case = W.make_attn_case(cfg, seed)
        got = run_oracle(case)
        ref = BR.brute_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache, case.block_table,
                                 case.ctx_lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale,
                                 block_size=case.block_size, num_flows=2, q_dtype=cfg.dtype,
                                 kv_dtype=cfg.dtype)
        for f in range(2):
            assert np.allclose(got[f"o{f + 1}"], np.array(ref[f]), rtol=0, atol=1e-12), (cfg.name, f)


def _sdpa(q, keys, values, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(keys)[None],
        torch.from_numpy(values)[None], scale=scale)
    return out[0, :, 0, :].numpy()


def pin_library_sdpa():
    """Flow 1 and (with a = 0) flow 2 equal torch SDPA, kv heads repeated for GQA."""
    for cfg, seed in TINY:
        case = W.make_attn_case(cfg, seed)
        case.a = np.zeros_like(case.a)
        got = run_oracle(case)
        q1 = W.bf16_bits_to_f32(case.q1) if cfg.dtype == "bf16" else case.q1
        q2 = W.bf16_bits_to_f32(case.q2) if cfg.dtype == "bf16" else case.q2
        dec = W.bf16_bits_to_f32 if cfg.dtype == "bf16" else (lambda x: x)
        for b in range(cfg.batch):
            n = int(case.ctx_lens[b])
            ks, vs = [], []
            for g in range(cfg.num_kv_heads):
                kr, vr = W.kv_rows(seed, b, g, n, cfg.head_dim, cfg.dtype, cfg.kv_std, cfg.peaky_fraction,
                                   cfg.peaky_factor)
                ks.append(dec(kr))
                vs.append(dec(vr))
            keys = np.repeat(np.stack(ks).astype(np.float64), cfg.group, axis=0)
            values = np.repeat(np.stack(vs).astype(np.float64), cfg.group, axis=0)
            for f, q in ((1, q1), (2, q2)):
                ref = _sdpa(q[b].astype(np.float64), keys, values, cfg.scale)
                assert np.allclose(got[f"o{f}"][b], ref, rtol=0, atol=1e-12), (cfg.name, b, f)


def _single(keys, values, q, scale=1.0):
    """Oracle on one sequence, one head, one flow, one f32 cache block."""
    keys = np.asarray(keys, dtype=np.float32)
    values = np.asarray(values, dtype=np.float32)
    n, d = keys.shape
    layout = W.plan_cache(1, np.array([n]), 0, 0, False, 0)
    k_cache, v_cache = W.empty_cache(layout, 1, d, "f32")
    W.store_rows(k_cache, v_cache, layout, 0, 0, keys, values)
    q = np.asarray(q, dtype=np.float32)[None, None]
    out = A.decode_attention(q, q, np.zeros((1, d), np.float32), k_cache, v_cache,
                             layout.block_table, np.array([n]), num_kv_heads=1, scale=scale,
                             block_size=layout.block_size, num_flows=2, q_dtype="f32", kv_dtype="f32",
                             return_weights=True)
    return out["o1"][0, 0], out["w"][(0, 0, 1)]


def pin_closed_forms():
    rng = np.random.default_rng(5)
    d = 8
    # one cached position: the output is that position's value
    v = rng.standard_normal((1, d)).astype(np.float32)
    o, _ = _single(rng.standard_normal((1, d)), v, rng.standard_normal(d))
    assert np.array_equal(o, v[0].astype(np.float64))
    # all keys zero: uniform weights, the output is the mean value
    vals = rng.standard_normal((7, d)).astype(np.float32)
    o, w = _single(np.zeros((7, d)), vals, rng.standard_normal(d))
    assert np.allclose(o, vals.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)
    # two keys: weights are the logistic function of the score difference
    keys = rng.standard_normal((2, d)).astype(np.float32)
    vals = rng.standard_normal((2, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    scale = 0.37
    s = scale * (keys.astype(np.float64) @ q.astype(np.float64))
    sig = 1.0 / (1.0 + math.exp(-(s[0] - s[1])))
    o, w = _single(keys, vals, q, scale)
    v64 = vals.astype(np.float64)
    assert np.allclose(o, sig * v64[0] + (1 - sig) * v64[1], rtol=0, atol=1e-14)
    # one key far dominant: the output is that key's value
    keys = rng.standard_normal((9, d)).astype(np.float32)
    vals = rng.standard_normal((9, d)).astype(np.float32)
    unit = q / np.linalg.norm(q)
    keys[4] = 400.0 * unit
    o, w = _single(keys, vals, unit)
    assert np.allclose(o, vals[4], rtol=0, atol=1e-12)


def pin_aux_equals_primary():
    for cfg, seed in TINY:
        case = W.make_attn_case(cfg, seed)
        case.q2 = case.q1.copy()
        case.a = np.zeros_like(case.a)
        got = run_oracle(case)
        assert np.array_equal(got["o1"], got["o2"]), cfg.name


def pin_weights_sum_to_one():
    for cfg, seed in TINY:
        case = W.make_attn_case(cfg, seed)
        got = run_oracle(case, return_weights=True)
        for (b, h, f), w in got["w"].items():
            assert w.shape == (int(case.ctx_lens[b]),)
            assert abs(w.sum() - 1.0) <= 1e-12 and np.all(w >= 0)


def pin_block_order():
    cfg, seed = TINY[0]
    case = W.make_attn_case(cfg, seed)
    ref = run_oracle(case)
    case.k_cache, case.v_cache, case.block_table = W.permute_blocks(case.k_cache, case.v_cache,
                                                                   case.block_table, 3)
    got = run_oracle(case)
    assert np.array_equal(ref["o1"], got["o1"]) and np.array_equal(ref["o2"], got["o2"])


def pin_key_shift():
    """Adding one vector to every key shifts all scores of a row equally: outputs unchanged."""
    cfg = W.AttnConfig("shift", batch=1, num_q_heads=2, num_kv_heads=1, head_dim=16, dtype="f32",
                       ctx_lens=(12,))
    case = W.make_attn_case(cfg, 4)
    case.k_cache = case.k_cache.astype(np.float64)  # the shift below is exact in float64
    case.v_cache = case.v_cache.astype(np.float64)
    ref = run_oracle(case, kv_dtype="f64")
    shift = 0.25 * np.arange(16, dtype=np.float64).reshape(2, 1, 8)  # dim 8*j+e lives at [.., j, :, e]
    case.k_cache = case.k_cache + shift
    got = run_oracle(case, kv_dtype="f64")
    assert np.allclose(ref["o1"], got["o1"], rtol=0, atol=1e-12)
    assert np.allclose(ref["o2"], got["o2"], rtol=0, atol=1e-12)


ALL_PINS = [pin_brute_force, pin_library_sdpa, pin_closed_forms, pin_aux_equals_primary,
            pin_weights_sum_to_one, pin_block_order, pin_key_shift]


def failing_pins():
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed
