"""GPU parity of dfa_prefill (primary-only prefill: cache write + causal attention) with oracle.prefill,
and of the auxiliary flow's first step at the last prompt position.

Bars: the cache after the prefill equals the oracle's bit for bit (slots past each prompt keep their
NaN fill); attention outputs within the row-normalised 2e-3 of the other GPU tests; rows past a
prompt are not written. The first auxiliary step (dfa_decode_attn over the written cache with
ctx_lens = prompt lengths) gives the primary's last prefill row for flow 1 and the oracle's
auxiliary output for flow 2. Cases: 1, 2, 4, 8 and 16 query heads per kv head, head_dim 64 and 128,
ragged prompts (lengths 0, 1, partial tiles, several query blocks and chunks), shuffled paged caches
with 16-, 32- and 64-position blocks, the full workload (4 prompts of 4096 tokens, 32/8 heads of
128: every row of the first prompt, sampled rows of the others), and the longest prompt the kernel
takes (2048 cache blocks).
"""
import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import TOL, assert_close, say
from oracle import attention as A
from oracle import prefill as PF
from workloads.device import to_device

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


def desc_of(case):
    cfg = case.cfg
    return dfa.PrefillDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                           head_dim=cfg.head_dim, max_prompt_len=case.q.shape[1], block_size=case.block_size,
                           max_blocks_per_seq=case.max_blocks_per_seq, num_blocks=case.k_cache.shape[0],
                           scale=cfg.scale)


def run_prefill(case):
    t = {name: to_device(getattr(case, name)) for name in ("q", "k", "v", "lens", "k_cache", "v_cache",
                                                            "block_table")}
    o = torch.full(case.q.shape, SENTINEL, dtype=torch.float32, device="cuda")
    dfa.dfa_prefill(desc_of(case), t["q"], t["k"], t["v"], t["lens"], t["k_cache"], t["v_cache"], t["block_table"], o)
    torch.cuda.synchronize()
    return t, o.cpu().numpy()


def cache_bits(x):
    return x.cpu().numpy().view(np.uint16)


def check_prefill(case, what):
    cfg = case.cfg
    t, o = run_prefill(case)
    ref_cache = PF.cache_after_prefill(case.k_cache, case.v_cache, case.block_table, case.k, case.v, case.lens,
                                       case.block_size)
    assert np.array_equal(cache_bits(t["k_cache"]), ref_cache["k_cache"]), f"{what}: key cache"
    assert np.array_equal(cache_bits(t["v_cache"]), ref_cache["v_cache"]), f"{what}: value cache"
    ref = PF.causal_attention(case.q, case.k, case.v, case.lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale)
    worst = 0.0
    for b in range(cfg.batch):
        n = int(case.lens[b])
        assert np.all(o[b, n:] == SENTINEL), f"{what}: rows past prompt {b} were written"
        if n:
            worst = max(worst, assert_close(o[b, :n], ref[b, :n], TOL, f"{what} prompt {b} (length {n})"))
    return t, o, ref_cache


CASES = {
    "g4_d128": (W.PrefillConfig("g4", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, lens=(1, 17, 100, 257)), 51),
    "g1_d64": (W.PrefillConfig("g1", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=64, lens=(200, 33),
                               block_size=32), 52),
    "g16_d128": (W.PrefillConfig("g16", batch=2, num_q_heads=16, num_kv_heads=1, head_dim=128, lens=(50, 8)), 53),
    "g8_d64": (W.PrefillConfig("g8", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=64, lens=(0, 95, 64),
                               block_size=64), 54),
    "g2_d128": (W.PrefillConfig("g2", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, lens=(300,),
                                shuffle_blocks=False), 55),
    "g4_d64": (W.PrefillConfig("g4d64", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64, lens=(161, 2),
                               block_size=32), 57),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    cfg, seed = CASES[name]
    case = W.make_prefill_case(cfg, seed)
    say(f"case prefill {name}: lengths {cfg.lens}, {cfg.num_q_heads}/{cfg.num_kv_heads} heads of {cfg.head_dim}")
    check_prefill(case, name)


def first_aux_step(case, t):
    """dfa_decode_attn at the last prompt position over the written cache (both flows)."""
    cfg = case.cfg
    last = np.stack([case.q[b, max(int(case.lens[b]) - 1, 0)] for b in range(cfg.batch)])
    d = dfa.AttnDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                     head_dim=cfg.head_dim, block_size=case.block_size, max_blocks_per_seq=case.max_blocks_per_seq,
                     num_blocks=case.k_cache.shape[0], max_ctx_len=int(case.lens.max()), num_flows=2, split_len=0,
                     scale=cfg.scale, q_dtype=dfa.DFA_BF16, kv_dtype=dfa.DFA_BF16)
    ws = torch.zeros(max(dfa.dfa_decode_attn_workspace_size(d) // 4, 4), device="cuda")
    o1 = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), device="cuda")
    o2 = torch.empty_like(o1)
    dfa.dfa_decode_attn(d, to_device(last), to_device(case.q2), to_device(case.a), t["k_cache"], t["v_cache"],
                        t["block_table"], t["lens"], ws, o1, o2)
    torch.cuda.synchronize()
    return last, o1.cpu().numpy(), o2.cpu().numpy()


def test_first_auxiliary_step_after_prefill():
    cfg = W.PrefillConfig("aux", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, lens=(129, 40, 300))
    case = W.make_prefill_case(cfg, 56)
    say("case prefill then the first auxiliary step")
    t, o, ref_cache = check_prefill(case, "aux")
    last, o1, o2 = first_aux_step(case, t)
    dec = A.decode_attention(last, case.q2, case.a.reshape(cfg.num_q_heads, cfg.head_dim), ref_cache["k_cache"],
                             ref_cache["v_cache"], case.block_table, case.lens, num_kv_heads=cfg.num_kv_heads,
                             scale=cfg.scale, block_size=case.block_size, num_flows=2, q_dtype="bf16",
                             kv_dtype="bf16")
    assert_close(o1, dec["o1"], TOL, "first step o1")
    assert_close(o2, dec["o2"], TOL, "first step o2 (auxiliary)")
    rows = np.stack([o[b, int(case.lens[b]) - 1] for b in range(cfg.batch)])
    assert_close(o1, rows, TOL, "first step o1 vs the prefill's last row")


def test_full_workload():
    cfg = W.PREFILL
    say("case prefill full size: generating inputs")
    case = W.make_prefill_case(cfg, W.SEEDS["prefill"])
    say("case prefill full size: running the GPU")
    t, o = run_prefill(case)
    assert np.all(np.isfinite(o))
    ref_cache = PF.cache_after_prefill(case.k_cache, case.v_cache, case.block_table, case.k, case.v, case.lens,
                                       case.block_size)
    assert np.array_equal(cache_bits(t["k_cache"]), ref_cache["k_cache"])
    assert np.array_equal(cache_bits(t["v_cache"]), ref_cache["v_cache"])
    # every row of the first prompt (4096 positions, 32 heads) against the causal oracle (~10 s)
    say("case prefill full size: causal oracle over every row of prompt 0")
    ref0 = PF.causal_attention(case.q[:1], case.k[:1], case.v[:1], case.lens[:1], num_kv_heads=cfg.num_kv_heads,
                               scale=cfg.scale)
    n0 = int(case.lens[0])
    assert_close(o[0, :n0], ref0[0, :n0], TOL, "prefill full prompt 0 (every row)")
    # rows of the other prompts: the attention of position t over [0, t] is the decode oracle with t + 1
    # cached positions
    for b, pos in ((1, 1), (2, 1000), (3, 4095), (3, 31)):
        lens = np.array([pos + 1], dtype=np.int32)
        ref = A.decode_attention(case.q[b, pos][None], None, None, ref_cache["k_cache"], ref_cache["v_cache"],
                                 case.block_table[b:b + 1], lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale,
                                 block_size=case.block_size, num_flows=1, q_dtype="bf16", kv_dtype="bf16")
        assert_close(o[b, pos], ref["o1"][0], TOL, f"prefill full b={b} t={pos}")
    last, o1, o2 = first_aux_step(case, t)
    rows = np.stack([o[b, int(case.lens[b]) - 1] for b in range(cfg.batch)])
    assert_close(o1, rows, TOL, "full first step o1 vs the prefill's last row")


def test_longest_prompt_fills_the_block_table():
    """A 32768-token prompt in 16-position blocks: 2048 block-table entries, the most the kernel stages
    (the host rejects one block more). Cache bit for bit, sampled rows against the decode oracle."""
    cfg = W.PrefillConfig("max", batch=1, num_q_heads=8, num_kv_heads=1, head_dim=128, lens=(32768,))
    say("case prefill: 32768 positions, 2048 cache blocks")
    case = W.make_prefill_case(cfg, 58)
    assert -(-int(case.lens.max()) // case.block_size) == 2048  # blocks the prompt spans (the table has a spare)
    t, o = run_prefill(case)
    assert np.all(np.isfinite(o))
    ref_cache = PF.cache_after_prefill(case.k_cache, case.v_cache, case.block_table, case.k, case.v, case.lens,
                                       case.block_size)
    assert np.array_equal(cache_bits(t["k_cache"]), ref_cache["k_cache"])
    assert np.array_equal(cache_bits(t["v_cache"]), ref_cache["v_cache"])
    for pos in (0, 15, 16, 4095, 16383, 16384, 32751, 32752, 32767):
        lens = np.array([pos + 1], dtype=np.int32)
        ref = A.decode_attention(case.q[0, pos][None], None, None, ref_cache["k_cache"], ref_cache["v_cache"],
                                 case.block_table, lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale,
                                 block_size=case.block_size, num_flows=1, q_dtype="bf16", kv_dtype="bf16")
        assert_close(o[0, pos], ref["o1"][0], TOL, f"prefill t={pos}")

