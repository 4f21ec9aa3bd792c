"""Input generators: determinism, bf16 encoding, cache layout."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_encoding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # plant exact ties
    u = x.view(np.uint32).copy()
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = u.view(np.float32)
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_seed_sensitive():
    cfg = W.C2.replace(batch=2, ctx_lens=(40, 40))
    a1 = W.make_attn_case(cfg, 5)
    a2 = W.make_attn_case(cfg, 5)
    a3 = W.make_attn_case(cfg, 6)
    for name in ("q1", "q2", "a", "k_cache", "v_cache"):
        assert np.array_equal(getattr(a1, name), getattr(a2, name))
    assert not np.array_equal(a1.q1, a3.q1)


def test_paged_layout_covers_each_sequence_once():
    cfg = W.C3.replace(batch=6, num_q_heads=16, ctx_range=(17, 70))
    case = W.make_attn_case(cfg, 3)
    assert np.all((case.ctx_lens >= 17) & (case.ctx_lens <= 70))
    used = case.block_table[case.block_table >= 0]
    assert len(np.unique(used)) == len(used) == case.k_cache.shape[0]
    for b in range(cfg.batch):
        n = -(-int(case.ctx_lens[b]) // 16)
        assert np.all(case.block_table[b, :n] >= 0) and np.all(case.block_table[b, n:] == -1)
    # unused slots hold NaN, used ones never do
    kv = W.bf16_bits_to_f32(case.k_cache)
    assert np.isnan(kv).sum() == (case.k_cache.shape[0] * 16 - case.ctx_lens.sum()) * cfg.num_kv_heads * cfg.head_dim


def test_logical_rows_land_where_the_table_says():
    cfg = W.C3.replace(batch=2, num_q_heads=16, ctx_range=(20, 40))
    case = W.make_attn_case(cfg, 9)
    b, g = 1, 3
    k_rows, v_rows = W.kv_rows(9, b, g, int(case.ctx_lens[b]), cfg.head_dim, "bf16")
    for t in range(int(case.ctx_lens[b])):
        blk = case.block_table[b, t // 16]
        assert np.array_equal(case.k_cache[blk, g, 0, :, t % 16, :].reshape(-1), k_rows[t])
        assert np.array_equal(case.v_cache[blk, g, 0, :, t % 16], v_rows[t])


def test_peaky_keys_scaled_by_eight():
    k0, _ = W.kv_rows(4, 0, 0, 1000, 8, "bf16")
    k1, _ = W.kv_rows(4, 0, 0, 1000, 8, "bf16", peaky_fraction=0.01, peaky_factor=8.0)
    f0, f1 = W.bf16_bits_to_f32(k0), W.bf16_bits_to_f32(k1)
    changed = np.where(np.any(f0 != f1, axis=1))[0]
    assert len(changed) == 10
    assert np.array_equal(f1[changed], 8 * f0[changed])


def test_permute_blocks_is_layout_only():
    cfg = W.C3.replace(batch=3, num_q_heads=16, ctx_range=(10, 50))
    case = W.make_attn_case(cfg, 2)
    k2, v2, t2 = W.permute_blocks(case.k_cache, case.v_cache, case.block_table, 1)
    for b in range(3):
        for t in range(int(case.ctx_lens[b])):
            j, s = divmod(t, 16)
            assert np.array_equal(case.k_cache[case.block_table[b, j], :, 0, :, s], k2[t2[b, j], :, 0, :, s])
            assert np.array_equal(case.v_cache[case.block_table[b, j], :, 0, :, s], v2[t2[b, j], :, 0, :, s])


def test_layer_case_shapes():
    cfg = W.C5.replace(batch=2, hidden=64, num_q_heads=4, num_kv_heads=2, head_dim=16, mlp=96, ctx=20, capacity=32)
    case = W.make_layer_case(cfg, 1)
    assert case.w["wq"].shape == (64, 64) and case.w["wk"].shape == (32, 64)
    assert case.w["wd"].shape == (64, 96)
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(case.x1)), case.x1)
    assert case.k_cache.shape == (2, 2, 2, 2, 16, 8) and case.v_cache.shape == (2, 2, 2, 16, 16)


def test_output_head_inputs_are_deterministic():
    cfg = W.MIX.replace(batch=5, vocab=64)
    a, b = W.make_mixture_case(cfg, 3), W.make_mixture_case(cfg, 3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert a[0].dtype == np.float32 and a[0].shape == (5, 64) and np.all((a[2] >= 0) & (a[2] < 1))
    assert not np.array_equal(a[0], a[1])  # the flows draw from separate streams
    h1, h2, w, u = W.make_head_case(W.HEAD.replace(batch=2, hidden=16, vocab=32), 4)
    assert w.dtype == np.uint16 and w.shape == (32, 16)
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(h1)), h1)  # exact bf16 values
