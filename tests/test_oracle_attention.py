"""The attention oracle against its pins, and the pins against planted mistakes."""
import numpy as np
import pytest

import attention_pins as P
from oracle import attention as A


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    pin()


def test_oracle_rejects_bad_inputs():
    cfg, seed = P.TINY[0]
    import workloads as W
    case = W.make_attn_case(cfg, seed)
    bad = case.block_table.copy()
    bad[1, 2] = -1  # a block the context needs
    with pytest.raises(ValueError):
        A.decode_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache, bad, case.ctx_lens,
                           num_kv_heads=2, scale=cfg.scale, block_size=16)
    with pytest.raises(ValueError):
        A.decode_attention(case.q1, case.q2, case.a, case.k_cache, case.v_cache, case.block_table,
                           np.array([0, 3]), num_kv_heads=2, scale=cfg.scale, block_size=16)


def test_pairs_subset_matches_full():
    cfg, seed = P.TINY[0]
    import workloads as W
    case = W.make_attn_case(cfg, seed)
    full = P.run_oracle(case)
    part = P.run_oracle(case, pairs=[(1, 0)])
    assert np.array_equal(full["o1"][1, :2], part["o1"][1, :2])
    assert np.isnan(part["o1"][0]).all() and np.isnan(part["o2"][1, 2:]).all()


# Plausible mistakes, each planted in the oracle; the pin battery must catch every one.
def _no_scale(q, keys, values, scale):
    w = A.softmax_weights(q @ keys.T)
    return w @ values, w


def _unnormalised(s):
    return np.exp(s - s.max(axis=-1, keepdims=True))


def _values_untransposed(v_cache, table_row, length, g, block_size, dtype):
    """Reads each transposed value tile as if it were [16 positions, D]."""
    blocks = A.block_rows(table_row, length, block_size)
    return A.to_f64(v_cache[blocks, g].reshape(-1, v_cache.shape[3])[:length], dtype)


_GATHER_KEYS = A.gather_keys


def _keys_rotated(k_cache, table_row, length, g, block_size, dtype):
    """Position t paired with the key of position t - 1."""
    return np.roll(_GATHER_KEYS(k_cache, table_row, length, g, block_size, dtype), 1, axis=0)


def _ignore_table(table_row, length, block_size):
    return np.arange(-(-length // block_size), dtype=np.int64)


MUTANTS = {
    "kv_head_interleaved": ("kv_head_of", lambda h, group: h % group),
    "coupling_dropped": ("coupled_query", lambda q1, q2, a: q2),
    "coupling_on_aux": ("coupled_query", lambda q1, q2, a: q2 + a * q2),
    "coupling_sign": ("coupled_query", lambda q1, q2, a: q2 - a * q1),
    "no_scale": ("attend", _no_scale),
    "unnormalised": ("softmax_weights", _unnormalised),
    "values_layout": ("gather_values", _values_untransposed),
    "keys_off_by_one": ("gather_keys", _keys_rotated),
    "ignores_block_table": ("block_rows", _ignore_table),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    assert P.failing_pins(), f"no pin caught the planted mistake {name}"
