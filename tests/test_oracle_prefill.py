"""Pins of oracle.prefill: brute force, torch's causal attention, the decode oracle at the last
prompt position, the cache gather of the attention oracle, invariants and planted mistakes."""
import math
import struct

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import formats as F
from oracle import prefill as PF

TINY = W.PrefillConfig("tiny", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8, lens=(5, 3), extra_slots=2)


def bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def run(case, **kw):
    cfg = case.cfg
    args = dict(q_bits=case.q, k_bits=case.k, v_bits=case.v, lens=case.lens)
    args.update(kw)
    return PF.causal_attention(**args, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale)


def brute(case):
    cfg = case.cfg
    g = cfg.num_q_heads // cfg.num_kv_heads
    out = {}
    for b in range(cfg.batch):
        for t in range(int(case.lens[b])):
            for h in range(cfg.num_q_heads):
                kv = h // g
                q = [bf16(x) for x in case.q[b, t, h]]
                s = [cfg.scale * math.fsum(qi * bf16(ki) for qi, ki in zip(q, case.k[b, u, kv])) for u in range(t + 1)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                out[b, t, h] = [math.fsum(w[u] / tot * bf16(case.v[b, u, kv, d]) for u in range(t + 1))
                                for d in range(cfg.head_dim)]
    return out


@pytest.mark.parametrize("cfg", [TINY, TINY.replace(num_kv_heads=4, lens=(4, 6)), TINY.replace(num_kv_heads=1)])
def test_brute_force(cfg):
    case = W.make_prefill_case(cfg, 3)
    got = run(case)
    for (b, t, h), ref in brute(case).items():
        assert np.max(np.abs(got[b, t, h] - np.array(ref))) <= 1e-12


def test_matches_torch_causal_attention():
    cfg = TINY.replace(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=16, lens=(37, 20))
    case = W.make_prefill_case(cfg, 4)
    got = run(case)
    g = cfg.num_q_heads // cfg.num_kv_heads
    for b in range(cfg.batch):
        n = int(case.lens[b])
        q = torch.from_numpy(F.to_f64(case.q[b, :n], "bf16")).permute(1, 0, 2)  # [H, n, D]
        k = torch.from_numpy(F.to_f64(case.k[b, :n], "bf16")).permute(1, 0, 2).repeat_interleave(g, 0)
        v = torch.from_numpy(F.to_f64(case.v[b, :n], "bf16")).permute(1, 0, 2).repeat_interleave(g, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=cfg.scale)
        assert np.max(np.abs(got[b, :n] - ref.permute(1, 0, 2).numpy())) <= 1e-12
        assert np.all(got[b, n:] == 0)


def test_last_position_is_the_decode_step_and_cache_holds_the_prompt():
    """The primary's last prompt row equals the decode oracle over the cache the prefill writes; the
    cache, read back through the decode oracle's own gather, holds the prompt's keys and values."""
    cfg = TINY.replace(batch=3, num_q_heads=6, num_kv_heads=2, head_dim=16, lens=(33, 17, 48), block_size=16)
    case = W.make_prefill_case(cfg, 5)
    got = run(case)
    c = PF.cache_after_prefill(case.k_cache, case.v_cache, case.block_table, case.k, case.v, case.lens,
                               case.block_size)
    for b in range(cfg.batch):
        n = int(case.lens[b])
        for g in range(cfg.num_kv_heads):
            kk = A.gather_keys(c["k_cache"], case.block_table[b], n, g, case.block_size, "bf16")
            vv = A.gather_values(c["v_cache"], case.block_table[b], n, g, case.block_size, "bf16")
            assert np.array_equal(kk, F.to_f64(case.k[b, :n, g], "bf16"))
            assert np.array_equal(vv, F.to_f64(case.v[b, :n, g], "bf16"))
    last = np.stack([case.q[b, int(case.lens[b]) - 1] for b in range(cfg.batch)])
    dec = A.decode_attention(last, case.q2, case.a.reshape(cfg.num_q_heads, cfg.head_dim), c["k_cache"],
                             c["v_cache"], case.block_table, case.lens, num_kv_heads=cfg.num_kv_heads,
                             scale=cfg.scale, block_size=case.block_size, num_flows=2, q_dtype="bf16",
                             kv_dtype="bf16")
    for b in range(cfg.batch):
        assert np.max(np.abs(dec["o1"][b] - got[b, int(case.lens[b]) - 1])) <= 1e-12


def test_invariants():
    cfg = TINY.replace(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8, lens=(9, 6))
    case = W.make_prefill_case(cfg, 6)
    got = run(case)
    # position 0 sees only itself: its value
    for b in range(cfg.batch):
        for h in range(cfg.num_q_heads):
            assert np.array_equal(got[b, 0, h], F.to_f64(case.v[b, 0, h // 2], "bf16"))
    # causality: a shorter prompt gives the same first rows
    short = run(case, lens=np.array([4, 2], dtype=np.int32))
    for b, n in enumerate((4, 2)):  # (matrix products of other sizes round differently)
        assert np.max(np.abs(short[b, :n] - got[b, :n])) <= 1e-14
    # later positions do not change earlier rows
    k2 = case.k.copy()
    k2[0, 7] = W.f32_to_bf16_bits(np.full(k2.shape[2:], 9.0, dtype=np.float32))
    changed = run(case, k_bits=k2)
    assert np.max(np.abs(changed[0, :7] - got[0, :7])) <= 1e-14
    assert np.max(np.abs(changed[0, 7:9] - got[0, 7:9])) > 1e-3


@pytest.mark.parametrize("mistake", ["not_causal", "strict_mask", "interleaved_heads", "no_scale"])
def test_planted_mistake_is_caught(mistake, monkeypatch):
    real = PF.causal_attention

    def planted(q_bits, k_bits, v_bits, lens, *, num_kv_heads, scale):
        q = F.to_f64(q_bits, "bf16")
        k = F.to_f64(k_bits, "bf16")
        v = F.to_f64(v_bits, "bf16")
        bsz, lmax, hq, d = q.shape
        group = hq // num_kv_heads
        out = np.zeros((bsz, lmax, hq, d))
        for b in range(bsz):
            n = int(lens[b])
            for h in range(hq):
                g = h % num_kv_heads if mistake == "interleaved_heads" else h // group
                s = (1.0 if mistake == "no_scale" else scale) * (q[b, :n, h] @ k[b, :n, g].T)
                if mistake == "strict_mask":
                    mask = np.tril(np.ones((n, n), dtype=bool), -1)
                    mask[0, 0] = True
                elif mistake == "not_causal":
                    mask = np.ones((n, n), dtype=bool)
                else:
                    mask = np.tril(np.ones((n, n), dtype=bool))
                s = np.where(mask, s, -np.inf)
                w = np.exp(s - s.max(axis=1, keepdims=True))
                out[b, :n, h] = (w / w.sum(axis=1, keepdims=True)) @ v[b, :n, g]
        return out

    monkeypatch.setattr(PF, "causal_attention", planted)
    checks = [lambda: test_brute_force(TINY), test_matches_torch_causal_attention,
              test_last_position_is_the_decode_step_and_cache_holds_the_prompt, test_invariants]
    failed = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed >= 1
    monkeypatch.setattr(PF, "causal_attention", real)
