"""dfa_decode_attn_noalloc (the allocation-free variant of dfa_decode_attn) against dfa_decode_attn.

The variant runs the same split plan and kernels with its split records in the
library's fixed device scratch instead of a caller workspace, so its outputs
must equal dfa_decode_attn's bit for bit, and both must meet the oracle's
2e-3 bar. Two calls in a row, the second with a smaller input (the scratch
keeps the first call's records; every record is rewritten), a third with 32
query rows per kv head, then a call whose records exceed the scratch: refused
on the host, nothing written.
"""
import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import TOL, assert_close, desc_for, oracle_attn, run_attn, say
from workloads.device import upload_attn_case

pytestmark = pytest.mark.gpu


def run_noalloc(case, split_len, desc=None):
    t = upload_attn_case(case)
    d = desc or desc_for(case, 2, split_len)
    B, H, D = case.cfg.batch, case.cfg.num_q_heads, case.cfg.head_dim
    o1 = torch.full((B, H, D), float("nan"), device="cuda")
    o2 = torch.full((B, H, D), float("nan"), device="cuda")
    dfa.dfa_decode_attn_noalloc(d, t["q1"], t["q2"], t["a"], t["k_cache"], t["v_cache"], t["block_table"],
                                t["ctx_lens"], o1, o2)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), o2.cpu().numpy()


CASES = [
    # several splits over a contiguous cache, with ragged lengths
    ("first", W.C2.replace(batch=6, ctx_lens=(4096, 3000, 17, 4000, 2049, 1), capacity=4096), 3101, 512),
    # a smaller input next: fewer sequences, fewer splits, paged and shuffled
    ("second", W.C3.replace(batch=3, num_q_heads=32, ctx_range=None, ctx_lens=(700, 33, 1500)), 3102, 256),
    # 32 query rows per kv head (two row sets), paged
    ("rows32", W.AttnConfig("r32", batch=2, num_q_heads=32, num_kv_heads=2, head_dim=128, dtype="bf16",
                            ctx_lens=(900, 2000), block_size=32, shuffle_blocks=True), 3103, 256),
]


def test_noalloc_matches_decode_attn_on_two_calls():
    for name, cfg, seed, split in CASES:
        case = W.make_attn_case(cfg, seed)
        d = desc_for(case, 2, split)
        ns = dfa.dfa_decode_attn_num_splits(d)
        need = dfa.dfa_decode_attn_workspace_size(d)
        say(f"case no-alloc {name}: batch {cfg.batch}, {ns} splits, records {need} bytes")
        assert ns > 1 and 0 < need <= 8 << 20
        got1, got2 = run_noalloc(case, split)
        ref1, ref2 = run_attn(case, num_flows=2, split_len=split)
        assert np.array_equal(got1, ref1) and np.array_equal(got2, ref2), f"{name}: differs from dfa_decode_attn"
        orc = oracle_attn(case)
        assert_close(got1, orc["o1"], TOL, f"no-alloc {name} o1")
        assert_close(got2, orc["o2"], TOL, f"no-alloc {name} o2")


def test_noalloc_refuses_records_beyond_the_scratch():
    # 64 sequences x 64 heads x 2 flows x 8 splits x 132 floats = 34.6 MB of records
    cfg = W.AttnConfig("big", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16",
                       ctx_lens=(64,) * 64, capacity=4096)
    case = W.make_attn_case(cfg, 3103)
    d = desc_for(case, 2, 32, max_ctx_len=256)
    assert dfa.dfa_decode_attn_workspace_size(d) > 8 << 20
    say("case no-alloc beyond the scratch")
    t = upload_attn_case(case)
    o1 = torch.full((64, 64, 128), float("nan"), device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    with pytest.raises(dfa.DfaError) as err:
        dfa.dfa_decode_attn_noalloc(d, t["q1"], t["q2"], t["a"], t["k_cache"], t["v_cache"], t["block_table"],
                                    t["ctx_lens"], o1, o2)
    assert "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert torch.isnan(o1).all() and torch.isnan(o2).all()
