"""The full-layer oracle against brute force, a library routine, and invariants."""
import numpy as np
import pytest
import scipy.special

import workloads as W
from oracle import brute as BR
from oracle import layer as LY

TINY = W.C5.replace(batch=2, hidden=16, num_q_heads=2, num_kv_heads=1, head_dim=8, mlp=24, ctx=20,
                    block_size=16, shuffle_blocks=True)


def run(case, **over):
    cfg = case.cfg
    args = dict(x1=case.x1, x2=case.x2, w=case.w, a=case.a, b=case.b, c=case.c,
                k_cache=case.k_cache, v_cache=case.v_cache, block_table=case.block_table,
                ctx_lens=case.ctx_lens)
    args.update(over)
    return LY.dual_flow_layer(**args, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                              head_dim=cfg.head_dim, scale=cfg.scale, block_size=case.block_size)


@pytest.mark.parametrize("cfg", [TINY, TINY.replace(block_size=0, capacity=16, ctx=7, num_kv_heads=2)])
def test_brute_force(cfg):
    case = W.make_layer_case(cfg, 21)
    got = run(case)
    ref = BR.brute_layer(case.x1, case.x2, case.w, case.a, case.b, case.c, case.k_cache, case.v_cache,
                         case.block_table, case.ctx_lens, num_q_heads=cfg.num_q_heads,
                         num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, scale=cfg.scale,
                         block_size=case.block_size)
    for key in ("o1", "o2", "out1", "out2"):
        assert np.allclose(got[key], np.array(ref[key]), rtol=0, atol=1e-12), key
    for key in ("k1_bits", "v1_bits"):
        assert np.array_equal(got[key].reshape(cfg.batch, -1), np.array(ref[key], dtype=np.uint16)), key


def test_silu_matches_library():
    u = np.linspace(-30, 30, 2001)
    assert np.allclose(LY.silu(u), u * scipy.special.expit(u), rtol=1e-15, atol=1e-300)


def test_aux_equals_primary_without_coupling():
    case = W.make_layer_case(TINY, 22)
    z = np.zeros_like
    got = run(case, x2=case.x1.copy(), a=z(case.a), b=z(case.b), c=z(case.c))
    assert np.array_equal(got["out1"], got["out2"]) and np.array_equal(got["o1"], got["o2"])


def test_zero_weights_return_the_input():
    case = W.make_layer_case(TINY, 23)
    w0 = {k: np.zeros_like(v) for k, v in case.w.items()}
    got = run(case, w=w0)
    assert np.array_equal(got["out1"], case.x1.astype(np.float64))
    assert np.array_equal(got["out2"], case.x2.astype(np.float64))


def test_primary_is_independent_of_the_aux_flow():
    case = W.make_layer_case(TINY, 24)
    ref = run(case)
    rng = np.random.default_rng(0)
    got = run(case, x2=rng.standard_normal(case.x2.shape).astype(np.float32),
              a=rng.standard_normal(case.a.shape), b=rng.standard_normal(case.b.shape),
              c=rng.standard_normal(case.c.shape))
    for key in ("q1", "k1", "v1", "o1", "h1", "z1", "m1", "out1", "k1_bits", "v1_bits", "k_cache", "v_cache"):
        assert np.array_equal(ref[key], got[key]), key
    assert not np.allclose(ref["out2"], got["out2"])


def test_append_writes_only_the_new_primary_slot():
    case = W.make_layer_case(TINY, 25)
    got = run(case)
    bs = case.block_size
    changed_k = np.argwhere(np.any(got["k_cache"] != case.k_cache, axis=(3, 5)))  # [blk, g, tile, s]
    expect = sorted((int(case.block_table[b, case.ctx_lens[b] // bs]), g, int(case.ctx_lens[b] % bs))
                    for b in range(TINY.batch) for g in range(TINY.num_kv_heads))
    assert sorted((int(i), int(g), int(t) * 16 + int(s)) for i, g, t, s in changed_k) == expect
    for b in range(TINY.batch):
        blk, slot = case.block_table[b, case.ctx_lens[b] // bs], case.ctx_lens[b] % bs
        assert np.array_equal(got["k_cache"][blk, :, slot // 16, :, slot % 16, :].reshape(TINY.num_kv_heads, -1),
                              got["k1_bits"][b])
        assert np.array_equal(got["v_cache"][blk, :, slot // 16, :, slot % 16], got["v1_bits"][b])
    changed_v = np.argwhere(np.any(got["v_cache"] != case.v_cache, axis=3))  # [blk, g, tile, s]
    assert sorted((int(i), int(g), int(t) * 16 + int(s)) for i, g, t, s in changed_v) == expect


def _brute_disagrees(cfg=TINY, seed=26):
    case = W.make_layer_case(cfg, seed)
    got = run(case)
    ref = BR.brute_layer(case.x1, case.x2, case.w, case.a, case.b, case.c, case.k_cache, case.v_cache,
                         case.block_table, case.ctx_lens, num_q_heads=cfg.num_q_heads,
                         num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, scale=cfg.scale,
                         block_size=case.block_size)
    same = all(np.allclose(got[k], np.array(ref[k]), rtol=0, atol=1e-12) for k in ("out1", "out2"))
    same &= all(np.array_equal(got[k].reshape(cfg.batch, -1), np.array(ref[k], dtype=np.uint16))
                for k in ("k1_bits", "v1_bits"))
    return not same


LAYER_MUTANTS = {
    "coupling_scales_aux": ("couple", lambda aux, vec, primary: aux + vec * aux),
    "coupling_dropped": ("couple", lambda aux, vec, primary: aux),
    "silu_is_sigmoid": ("silu", lambda u: 1.0 / (1.0 + np.exp(-u))),
    "kv_rounding_truncates": ("f64_to_bf16_bits",
                              lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)),
}


@pytest.mark.parametrize("name", sorted(LAYER_MUTANTS))
def test_planted_layer_mistake_is_caught(name, monkeypatch):
    attr, fn = LAYER_MUTANTS[name]
    monkeypatch.setattr(LY, attr, fn)
    assert _brute_disagrees()
