"""GPU parity of dfa_decode_attn / dfa_decode_attn_partials / dfa_combine with the oracle.

Element-by-element against the float64 oracle on reduced shapes of each
workload (several 32-position chunks, several splits, ragged tails, paged and
contiguous caches, G in {1, 2, 4, 8, 12, 16, 32}, up to 32 query rows per kv head); every
(sequence, kv head) pair at the full workload sizes in the benchmark's launch configuration; and the
invariants the method fixes (primary independence, the cache is never written,
aux == primary without coupling, one position returns its value, paging and
split plans do not change the result). Unused cache slots hold NaN, so any read
past a sequence shows up as a non-finite output.
"""
import copy

import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import TOL, assert_close, desc_for, oracle_attn, run_attn, say
from workloads.device import upload_attn_case

pytestmark = pytest.mark.gpu

SMALL = {
    "c1": (W.C1, 1001),
    "c2_ragged": (W.C2.replace(batch=3, ctx_lens=(1000, 4096, 37), capacity=4096), 2002),
    "c3_paged": (W.C3.replace(batch=6, ctx_range=None, ctx_lens=(1, 17, 33, 700, 1024, 513)), 2003),
    "c4_peaky": (W.C4.replace(batch=1, ctx_lens=(20000,)), 2004),
    "c5_f32q": (W.C2.replace(batch=2, ctx_lens=(4097, 4097), capacity=8192, q_dtype="f32"), 2005),
    "d64": (W.AttnConfig("d64", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64, dtype="bf16",
                         ctx_lens=(300, 65)), 2006),
    "g2_paged": (W.AttnConfig("g2", batch=2, num_q_heads=8, num_kv_heads=4, head_dim=128, dtype="bf16",
                              ctx_lens=(90, 31), block_size=32, shuffle_blocks=True), 2007),
    "mha_bf16": (W.AttnConfig("mha", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128, dtype="bf16",
                              ctx_lens=(64, 200)), 2008),
    "f32_d128_g4": (W.AttnConfig("f32g4", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="f32",
                                 ctx_lens=(129, 700), block_size=64, shuffle_blocks=True), 2009),
    # 16 query rows per workgroup (8 heads x 2 flows) at head_dim 64, and with float32 queries
    "d64_rows16": (W.AttnConfig("d64r16", batch=2, num_q_heads=32, num_kv_heads=4, head_dim=64, dtype="bf16",
                                ctx_lens=(513, 96), block_size=32, shuffle_blocks=True), 2015),
    "f32q_rows16": (W.AttnConfig("f32qr16", batch=2, num_q_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16",
                                 ctx_lens=(1025, 40), capacity=2048, q_dtype="f32"), 2016),
    # more than 16 rows per kv head: a second row set of waves (16 heads x 2 flows; 12 heads x 2 flows)
    "g16_paged": (W.AttnConfig("g16p", batch=3, num_q_heads=32, num_kv_heads=2, head_dim=128, dtype="bf16",
                               ctx_lens=(600, 4097, 33), block_size=32, shuffle_blocks=True), 2018),
    "g16_d64_f32q": (W.AttnConfig("g16d64", batch=2, num_q_heads=16, num_kv_heads=1, head_dim=64, dtype="bf16",
                                  ctx_lens=(257, 1000), q_dtype="f32"), 2019),
    "g12": (W.AttnConfig("g12", batch=2, num_q_heads=36, num_kv_heads=3, head_dim=128, dtype="bf16",
                         ctx_lens=(100, 513)), 2020),
    # more than 64 sequences: one split each, taken in batch order (no length ranking)
    "batch70": (W.AttnConfig("b70", batch=70, num_q_heads=8, num_kv_heads=4, head_dim=128, dtype="bf16",
                             ctx_range=(1, 300), block_size=16, shuffle_blocks=True), 2017),
}
_CASES = {}
_REFS = {}


def small_case(name):
    if name not in _CASES:
        cfg, seed = SMALL[name]
        _CASES[name] = W.make_attn_case(cfg, seed)
    return _CASES[name]


def small_ref(name, flows):
    if (name, flows) not in _REFS:
        _REFS[(name, flows)] = oracle_attn(small_case(name), num_flows=flows)
    return _REFS[(name, flows)]


@pytest.mark.parametrize("split", [0, 32, 256, 4096])
@pytest.mark.parametrize("flows", [2, 1])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_parity_small(name, flows, split):
    case = small_case(name)
    say(f"case {name} flows={flows} split={split}")
    o1, o2 = run_attn(case, num_flows=flows, split_len=split)
    ref = small_ref(name, flows)
    assert_close(o1, ref["o1"], what=f"{name} o1")
    if flows == 2:
        assert_close(o2, ref["o2"], what=f"{name} o2")


def test_groups_of_16_and_32():
    """16 heads per kv head: one row set with one flow, two with both flows, and the primary bit for bit
    the same either way; 32 heads per kv head with one flow (32 rows); 64 rows are refused."""
    cfg = W.AttnConfig("g16", batch=2, num_q_heads=32, num_kv_heads=2, head_dim=128, dtype="bf16",
                       ctx_lens=(77, 300))
    case = W.make_attn_case(cfg, 2010)
    say("case g16 one flow, two flows")
    ref = oracle_attn(case)
    for split in (64, 0):
        p1, _ = run_attn(case, num_flows=1, split_len=split)
        o1, o2 = run_attn(case, num_flows=2, split_len=split)
        assert_close(p1, ref["o1"], what=f"g16 split {split} one-flow o1")
        assert_close(o1, ref["o1"], what=f"g16 split {split} o1")
        assert_close(o2, ref["o2"], what=f"g16 split {split} o2")
        assert np.array_equal(p1, o1), "the primary must not depend on the second row set"
    cfg32 = W.AttnConfig("g32", batch=2, num_q_heads=32, num_kv_heads=1, head_dim=64, dtype="bf16",
                         ctx_lens=(129, 40))
    case32 = W.make_attn_case(cfg32, 2011)
    say("case g32 one flow")
    o1, _ = run_attn(case32, num_flows=1, split_len=64)
    assert_close(o1, oracle_attn(case32, num_flows=1)["o1"], what="g32 o1")
    with pytest.raises(dfa.DfaError):  # 32 heads x 2 flows exceed a workgroup's 32 rows
        run_attn(case32, num_flows=2)


# ---------------------------------------------------------------- full sizes
FULL = {"c2": W.C2, "c3": W.C3, "c4": W.C4, "g16": W.G16}


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "g16"])
def test_full_size_all_pairs(name):
    """Every output row of the full workload, in the benchmark's launch configuration (the
    library's plan), against the oracle."""
    cfg = FULL[name]
    say(f"case {name} full size: generating inputs")
    case = W.make_attn_case(cfg, W.SEEDS[name], pad_nan=True)
    d = desc_for(case, 2, 0)
    say(f"case {name}: kv {case.k_cache.nbytes * 2 / 2**30:.2f} GiB, {dfa.dfa_decode_attn_num_splits(d)} "
        f"split(s) per sequence; running the GPU")
    o1, o2 = run_attn(case, num_flows=2, split_len=0)
    say(f"case {name}: oracle over all {cfg.batch * cfg.num_kv_heads} (sequence, kv head) pairs")
    ref = oracle_attn(case)
    assert_close(o1, ref["o1"], what=f"{name} o1")
    assert_close(o2, ref["o2"], what=f"{name} o2")


# ---------------------------------------------------------------- invariants
def test_primary_independent_of_aux_inputs():
    case = small_case("c3_paged")
    t = upload_attn_case(case)
    say("case primary independence")
    o1a, o2a = run_attn(case, tensors=t)
    gen = torch.Generator(device="cpu").manual_seed(77)
    # scales 1 and 16: large auxiliary scores move the auxiliary rows' running max on chunks
    # where the primary rows keep theirs; the primary must stay bit for bit the same
    for scale in (1.0, 16.0):
        q2 = torch.randn(t["q2"].shape, generator=gen) * scale
        t["q2"] = q2.to(torch.bfloat16).view(torch.int16).cuda()
        t["a"] = (torch.randn(t["a"].shape, generator=gen) * scale).cuda()
        o1b, o2b = run_attn(case, tensors=t)
        assert np.array_equal(o1a, o1b), f"aux scale {scale}"
        assert not np.array_equal(o2a, o2b)


def test_cache_is_never_written():
    case = small_case("c2_ragged")
    t = upload_attn_case(case)
    k0, v0 = t["k_cache"].clone(), t["v_cache"].clone()
    say("case cache read-only")
    run_attn(case, tensors=t, split_len=256)
    run_attn(case, tensors=t, split_len=0)
    assert torch.equal(k0, t["k_cache"]) and torch.equal(v0, t["v_cache"])


@pytest.mark.parametrize("name", ["c2_ragged", "c3_paged", "c1"])
def test_aux_equals_primary_without_coupling(name):
    case = small_case(name)
    t = upload_attn_case(case)
    t["q2"] = t["q1"].clone()
    t["a"] = torch.zeros_like(t["a"])
    say(f"case aux==primary {name}")
    o1, o2 = run_attn(case, tensors=t, split_len=256)
    assert np.array_equal(o1, o2)


def test_one_position_returns_its_value():
    cfg = W.C2.replace(batch=2, ctx_lens=(1, 1), capacity=32)
    case = W.make_attn_case(cfg, 2011)
    say("case length-1 context")
    o1, o2 = run_attn(case)
    v = W.bf16_bits_to_f32(case.v_cache[:, :, 0, :, 0])  # position 0 of each sequence: [B, Hkv, D]
    expect = np.repeat(v, cfg.group, axis=1)
    assert np.array_equal(o1, expect) and np.array_equal(o2, expect)


def test_constant_values_return_that_value():
    case = W.make_attn_case(W.C2.replace(batch=2, ctx_lens=(777, 2048), capacity=2048), 2012)
    vconst = W.f32_to_bf16_bits(np.linspace(-2, 2, 128, dtype=np.float32))
    case.v_cache[...] = vconst[None, None, None, :, None]  # every position holds vconst
    say("case constant values")
    o1, o2 = run_attn(case, split_len=256)
    expect = W.bf16_bits_to_f32(vconst)[None, None, :]
    assert np.abs(o1 - expect).max() <= 1e-5 * 2 and np.abs(o2 - expect).max() <= 1e-5 * 2


def test_physical_block_order_does_not_matter():
    case = small_case("c3_paged")
    say("case block permutation")
    o1a, o2a = run_attn(case, split_len=64)
    case2 = W.make_attn_case(SMALL["c3_paged"][0], SMALL["c3_paged"][1])
    case2.k_cache, case2.v_cache, case2.block_table = W.permute_blocks(case2.k_cache, case2.v_cache,
                                                                      case2.block_table, 5)
    o1b, o2b = run_attn(case2, split_len=64)
    assert np.array_equal(o1a, o1b) and np.array_equal(o2a, o2b)


def test_paged_equals_contiguous():
    """The same sequences in 16-position blocks (shuffled) and in one block each give the same bits."""
    cfg = W.C2.replace(batch=3, ctx_lens=(100, 333, 64), capacity=512)
    contiguous = W.make_attn_case(cfg, 2013)
    paged = W.make_attn_case(cfg.replace(block_size=16, shuffle_blocks=True), 2013)
    say("case paged vs contiguous")
    assert np.array_equal(W.bf16_bits_to_f32(contiguous.q1), W.bf16_bits_to_f32(paged.q1))
    a1, a2 = run_attn(contiguous, split_len=128)
    b1, b2 = run_attn(paged, split_len=128)
    assert np.array_equal(a1, b1) and np.array_equal(a2, b2)


def test_gqa_equals_mha_with_repeated_kv_heads():
    """Grouped-query attention is multi-head attention with each kv head repeated G times."""
    gqa = W.make_attn_case(W.C2.replace(batch=2, num_q_heads=8, num_kv_heads=2, ctx_lens=(300, 77),
                                        capacity=512), 2014)
    mha = copy.copy(gqa)
    mha.cfg = gqa.cfg.replace(num_kv_heads=8)
    mha.k_cache = np.ascontiguousarray(np.repeat(gqa.k_cache, 4, axis=1))
    mha.v_cache = np.ascontiguousarray(np.repeat(gqa.v_cache, 4, axis=1))
    say("case gqa vs repeated-kv mha")
    g1, g2 = run_attn(gqa, split_len=128)
    m1, m2 = run_attn(mha, split_len=128)
    # rows share a wave-wide rescale decision, so the two layouts may round differently
    assert_close(m1, g1, tol=1e-6, what="mha o1 vs gqa o1")
    assert_close(m2, g2, tol=1e-6, what="mha o2 vs gqa o2")


def test_split_plans_agree():
    case = small_case("c4_peaky")
    say("case split plans")
    outs = [run_attn(case, split_len=s) for s in (32, 256, 2048, 20000)]
    for o1, o2 in outs[1:]:
        assert_close(o1, outs[0][0], tol=1e-4, what="o1 vs split 32")
        assert_close(o2, outs[0][1], tol=1e-4, what="o2 vs split 32")


def test_one_flow_matches_two_flow_primary():
    for name in ("c2_ragged", "c3_paged"):
        case = small_case(name)
        say(f"case flows 1 vs 2 {name}")
        o1_two, _ = run_attn(case, num_flows=2, split_len=256)
        o1_one, _ = run_attn(case, num_flows=1, split_len=256)
        if case.cfg.group * 2 <= 8:  # same packing: identical arithmetic per row
            assert np.array_equal(o1_one, o1_two)
        else:
            assert_close(o1_one, o1_two, tol=1e-4, what=f"{name} o1 one vs two flows")


def test_partials_then_combine_equals_decode_attn():
    case = small_case("c2_ragged")
    t = upload_attn_case(case)
    d = desc_for(case, split_len=128)
    say("case partials + combine")
    o1, o2 = run_attn(case, tensors=t, desc=d)
    ws = torch.zeros(dfa.dfa_decode_attn_workspace_size(d) // 4, dtype=torch.float32, device="cuda")
    p1 = torch.full_like(torch.from_numpy(o1), float("nan")).cuda()
    p2 = torch.full_like(p1, float("nan"))
    dfa.dfa_decode_attn_partials(d, t["q1"], t["q2"], t["a"], t["k_cache"], t["v_cache"], t["block_table"],
                                 t["ctx_lens"], ws)
    dfa.dfa_combine(d, ws, p1, p2)
    torch.cuda.synchronize()
    # the same splits and merge; a one-split sequence is normalised as o / l by the fused
    # kernel and as o * (1 / l) by dfa_combine, so allow rounding
    assert_close(p1.cpu().numpy(), o1, tol=1e-6, what="partials+combine o1")
    assert_close(p2.cpu().numpy(), o2, tol=1e-6, what="partials+combine o2")
    # a record holds (O, m, l): O / l of a one-split plan is the output
    d1 = desc_for(case, split_len=4096)
    ws1 = torch.zeros(dfa.dfa_decode_attn_workspace_size(d1) // 4, dtype=torch.float32, device="cuda")
    dfa.dfa_decode_attn_partials(d1, t["q1"], t["q2"], t["a"], t["k_cache"], t["v_cache"], t["block_table"],
                                 t["ctx_lens"], ws1)
    torch.cuda.synchronize()
    rec = ws1.cpu().numpy().reshape(3, 32, 2, 1, 132)
    d1o1, d1o2 = run_attn(case, tensors=t, desc=d1)  # the same one-split plan, normalised in the kernel
    assert_close(rec[:, :, 0, 0, :128] / rec[:, :, 0, 0, 129:130], d1o1, tol=1e-6, what="record O/l flow 1")
    assert_close(rec[:, :, 1, 0, :128] / rec[:, :, 1, 0, 129:130], d1o2, tol=1e-6, what="record O/l flow 2")


def test_empty_sequence_gives_zeros():
    case = small_case("c2_ragged")
    t = upload_attn_case(case)
    t["ctx_lens"][1] = 0
    say("case empty sequence")
    for split in (256, 4096):
        o1, o2 = run_attn(case, tensors=t, split_len=split)
        assert np.all(o1[1] == 0) and np.all(o2[1] == 0)
        assert np.all(np.isfinite(o1)) and np.all(np.isfinite(o2))


def test_workspace_reuse_across_split_plans():
    """One workspace serves calls with different split plans in a row."""
    case = small_case("c3_paged")
    t = upload_attn_case(case)
    ref = small_ref("c3_paged", 2)
    big = dfa.dfa_decode_attn_workspace_size(desc_for(case, split_len=32))
    ws = torch.full((big // 4,), float("nan"), dtype=torch.float32, device="cuda")
    for split in (32, 256, 64, 0, 32):
        d = desc_for(case, split_len=split)
        o1 = torch.full((6, 64, 128), float("nan"), device="cuda")
        o2 = torch.full_like(o1, float("nan"))
        say(f"case workspace reuse split={split}")
        dfa.dfa_decode_attn(d, t["q1"], t["q2"], t["a"], t["k_cache"], t["v_cache"], t["block_table"],
                            t["ctx_lens"], ws, o1, o2)
        torch.cuda.synchronize()
        assert_close(o1.cpu().numpy(), ref["o1"], what=f"split {split} o1")
        assert_close(o2.cpu().numpy(), ref["o2"], what=f"split {split} o2")


def test_timed_call_matches_untimed():
    case = small_case("c2_ragged")
    t = upload_attn_case(case)
    for split in (256, 4096):
        d = desc_for(case, split_len=split)
        ws = torch.empty(max(dfa.dfa_decode_attn_workspace_size(d) // 4, 4), dtype=torch.float32, device="cuda")
        o1, o2 = run_attn(case, tensors=t, desc=d)
        p1 = torch.empty((3, 32, 128), device="cuda")
        p2 = torch.empty_like(p1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        say(f"case timed call split={split}")
        dfa.dfa_decode_attn_timed(d, t["q1"], t["q2"], t["a"], t["k_cache"], t["v_cache"], t["block_table"],
                                  t["ctx_lens"], ws, p1, p2, start=e0, stop=e1)
        torch.cuda.synchronize()
        assert np.array_equal(p1.cpu().numpy(), o1) and np.array_equal(p2.cpu().numpy(), o2)
        ms = e0.elapsed_time(e1)
        assert 0 < ms < 100, ms
