"""The C ABI on the host: the library loads, exports what include/dfa.h declares,
plans splits, and rejects invalid calls before enqueuing anything.

None of these calls reaches a kernel launch: every call with device pointers
here fails host-side validation (the pointers are never dereferenced).
"""
import ctypes
import math
import os
import re

import pytest

import dual_flow_shared_decode_amd as dfa
from dual_flow_shared_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # an aligned, never-dereferenced stand-in for a device address


def c2_desc(**kw):
    d = dict(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=4096,
             max_blocks_per_seq=1, num_blocks=16, max_ctx_len=4096, num_flows=2, split_len=0,
             scale=1 / math.sqrt(128), q_dtype=dfa.DFA_BF16, kv_dtype=dfa.DFA_BF16)
    d.update(kw)
    return dfa.AttnDesc(**d)


def test_header_declarations_are_exported():
    with open(os.path.join(ROOT, "include", "dfa.h")) as f:
        header = f.read()
    declared = set(re.findall(r"DFA_API\s+[\w\s\*]+?\b(dfa_\w+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    L = dfa.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings_and_version():
    for code in range(8):
        assert dfa.dfa_status_string(code)
    assert dfa.dfa_version() >= 100


def test_split_plan_and_workspace_size():
    d = c2_desc()
    split = dfa.dfa_decode_attn_split_len(d)
    ns = dfa.dfa_decode_attn_num_splits(d)
    assert split % 32 == 0 and ns == -(-4096 // split)
    assert dfa.dfa_decode_attn_workspace_size(d) == 16 * 32 * 2 * ns * (128 + 4) * 4
    # about 256 workgroups: 128 (sequence, kv head) pairs take 2 splits, 32 pairs 8, 256 pairs 1
    assert ns == 2 and split == 2048
    d4 = c2_desc(batch=4, block_size=131072, max_ctx_len=131072)
    assert dfa.dfa_decode_attn_split_len(d4) == 16384 and dfa.dfa_decode_attn_num_splits(d4) == 8
    assert dfa.dfa_decode_attn_num_splits(c2_desc(batch=32)) == 1
    # short contexts: splits never go below 512 positions
    assert dfa.dfa_decode_attn_split_len(c2_desc(batch=1, block_size=1024, max_ctx_len=1000)) == 512
    d1 = c2_desc(split_len=4096)
    assert dfa.dfa_decode_attn_num_splits(d1) == 1
    assert dfa.dfa_decode_attn_split_len(c2_desc(split_len=96)) == 96


def test_row_limits():
    """Up to 32 query rows (heads per kv head x flows) with a bf16 cache, 16 with a float32 cache."""
    plan = lambda **kw: _lib.lib().dfa_decode_attn_split_len(ctypes.byref(c2_desc(**kw)))
    for hq, flows in ((128, 2), (256, 1), (72, 2), (64, 2)):
        assert plan(num_q_heads=hq, num_flows=flows) > 0
    assert _lib.STATUS[-plan(num_q_heads=256, num_flows=2)] == "DFA_ERR_UNSUPPORTED"
    f32 = dict(q_dtype=dfa.DFA_F32, kv_dtype=dfa.DFA_F32)
    assert plan(num_q_heads=64, **f32) > 0
    assert plan(num_q_heads=128, num_flows=1, **f32) > 0
    assert _lib.STATUS[-plan(num_q_heads=128, **f32)] == "DFA_ERR_UNSUPPORTED"


@pytest.mark.parametrize("change,status", [
    (dict(batch=0), "DFA_ERR_SHAPE"),
    (dict(num_q_heads=30), "DFA_ERR_SHAPE"),
    (dict(num_flows=3), "DFA_ERR_SHAPE"),
    (dict(head_dim=96), "DFA_ERR_UNSUPPORTED"),
    (dict(num_q_heads=136), "DFA_ERR_UNSUPPORTED"),  # 17 heads per kv head x 2 flows > 32 rows
    (dict(num_q_heads=72, q_dtype=dfa.DFA_F32, kv_dtype=dfa.DFA_F32), "DFA_ERR_UNSUPPORTED"),  # > 16 rows, f32 cache
    (dict(block_size=48), "DFA_ERR_SHAPE"),
    (dict(block_size=8, max_blocks_per_seq=512), "DFA_ERR_SHAPE"),
    (dict(max_ctx_len=0), "DFA_ERR_SHAPE"),
    (dict(max_ctx_len=4097), "DFA_ERR_SHAPE"),  # beyond max_blocks_per_seq * block_size
    (dict(split_len=100), "DFA_ERR_SHAPE"),
    (dict(scale=float("nan")), "DFA_ERR_SHAPE"),
    (dict(q_dtype=dfa.DFA_BF16, kv_dtype=dfa.DFA_F32), "DFA_ERR_DTYPE"),
    (dict(kv_dtype=7), "DFA_ERR_DTYPE"),
    (dict(block_size=16, max_blocks_per_seq=256, split_len=16384 + 32), "DFA_ERR_UNSUPPORTED"),
])
def test_invalid_descriptors(change, status):
    d = c2_desc(**change)
    v = _lib.lib().dfa_decode_attn_split_len(ctypes.byref(d))
    assert v < 0 and _lib.STATUS[-v] == status
    assert dfa.dfa_decode_attn_workspace_size(d) == 0
    with pytest.raises(dfa.DfaError) as e:
        _call_attn(d)
    assert _lib.STATUS[e.value.status] == status
    assert _lib.lib().dfa_last_error().decode()


def _call_attn(d, **ptrs):
    p = dict(q1=FAKE, q2=FAKE, a=FAKE, k=FAKE, v=FAKE, table=FAKE, ctx=FAKE, ws=FAKE, ws_bytes=0,
             o1=FAKE, o2=FAKE)
    p.update(ptrs)
    st = _lib.lib().dfa_decode_attn(ctypes.byref(d), p["q1"], p["q2"], p["a"], p["k"], p["v"], p["table"],
                                    p["ctx"], p["ws"], p["ws_bytes"], p["o1"], p["o2"], None)
    _lib._check(st)


@pytest.mark.parametrize("missing", ["q1", "k", "v", "table", "ctx", "o1", "q2", "a", "o2"])
def test_null_pointers(missing):
    with pytest.raises(dfa.DfaError) as e:
        _call_attn(c2_desc(), **{missing: None})
    assert _lib.STATUS[e.value.status] == "DFA_ERR_NULL"


def test_single_flow_accepts_null_aux_pointers_until_the_workspace_check():
    with pytest.raises(dfa.DfaError) as e:  # split_len 512: several splits, so a workspace is needed
        _call_attn(c2_desc(num_flows=1, split_len=512), q2=None, a=None, o2=None, ws=None)
    assert _lib.STATUS[e.value.status] == "DFA_ERR_WORKSPACE"


def test_workspace_and_alignment_errors():
    d = c2_desc(split_len=512)  # several splits, so a workspace is needed
    need = dfa.dfa_decode_attn_workspace_size(d)
    with pytest.raises(dfa.DfaError) as e:
        _call_attn(d, ws=None)
    assert _lib.STATUS[e.value.status] == "DFA_ERR_WORKSPACE"
    with pytest.raises(dfa.DfaError) as e:
        _call_attn(d, ws_bytes=need - 4)
    assert _lib.STATUS[e.value.status] == "DFA_ERR_WORKSPACE"
    for name in ("q1", "k", "ws", "o1", "a"):
        with pytest.raises(dfa.DfaError) as e:
            _call_attn(d, ws_bytes=need - 4, **{name: FAKE + 4})
        assert _lib.STATUS[e.value.status] == "DFA_ERR_ALIGNMENT", name
    with pytest.raises(dfa.DfaError) as e:
        _lib._check(_lib.lib().dfa_combine(ctypes.byref(d), FAKE, need - 4, FAKE, FAKE, None))
    assert _lib.STATUS[e.value.status] == "DFA_ERR_WORKSPACE"
    with pytest.raises(dfa.DfaError) as e:
        _lib._check(_lib.lib().dfa_decode_attn_partials(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                        FAKE, None, 0, None))
    assert _lib.STATUS[e.value.status] == "DFA_ERR_WORKSPACE"


def test_stream_read_validation():
    with pytest.raises(dfa.DfaError):
        _lib._check(_lib.lib().dfa_stream_read(FAKE, 100, FAKE, None))
    with pytest.raises(dfa.DfaError):
        _lib._check(_lib.lib().dfa_stream_read(None, 1024, FAKE, None))
    assert dfa.dfa_stream_read_sink_bytes() > 0


def gemv_desc(**kw):
    d = dict(batch=32, n=4096, k=4096, num_flows=2, epilogue=0, x_exact_bf16=0, k_split=0, rows_per_wg=0)
    d.update(kw)
    return dfa.GemvDesc(**d)


def test_gemv_plans():
    """The library's GEMV plans at the layer's shapes (batch 32, two flows: 64 padded rows)."""
    rows = 2 * 32
    # 4096 x 4096: 64-row workgroups, 64 row groups -> 4 k-splits
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc()) == 4 * rows * 4096 * 4
    # 4096 x 14336 (MLP down): 128-row workgroups, 32 row groups -> 8 k-splits
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(k=14336)) == 8 * rows * 4096 * 4
    # forced 64 rows: 64 row groups -> 4 k-splits
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(k=14336, rows_per_wg=64)) == 4 * rows * 4096 * 4
    # 14336 x 4096 SwiGLU pair: 224 row groups of 64 rows run unsplit (no workspace)
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=14336, epilogue=dfa.DFA_EPI_SWIGLU)) == 0
    # KV append, one flow (32 padded rows), 1024 columns: 16 row groups -> 16 k-splits of two matrices
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=1024, num_flows=1, epilogue=dfa.DFA_EPI_KV_APPEND)) == \
        16 * 2 * 32 * 1024 * 4
    # 64 x 4096 (MoE router): one row group; the library's choice stops at 16 k-splits
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=64)) == 16 * rows * 64 * 4
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=64, k_split=32)) == 32 * rows * 64 * 4
    # 32000 x 4096 (output head over the vocabulary): 250 row groups of 128 rows, unsplit
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=32000)) == 0
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=32000, rows_per_wg=64, k_split=2)) == 2 * rows * 32000 * 4
    # invalid: rows_per_wg not 0/64/128, or 128 with n % 128 != 0
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(rows_per_wg=96)) == 0
    assert dfa.dfa_dual_gemv_workspace_size(gemv_desc(n=192, rows_per_wg=128)) == 0


def test_mixture_workspace_and_validation():
    d = dfa.MixtureDesc(batch=32, vocab=32000)
    # per (sequence, chunk of 4096 tokens): 8 floats of softmax statistics and 4 words of mass and maximum
    assert dfa.dfa_mixture_workspace_size(d) == 32 * 8 * (32 + 16)
    assert dfa.dfa_mixture_workspace_size(dfa.MixtureDesc(batch=1, vocab=1 << 20)) == 256 * 48
    for bad in (dict(batch=0, vocab=32000), dict(batch=65536, vocab=32000), dict(batch=1, vocab=0),
                dict(batch=1, vocab=30), dict(batch=1, vocab=2), dict(batch=1, vocab=(1 << 20) + 4)):
        assert dfa.dfa_mixture_workspace_size(dfa.MixtureDesc(**bad)) == 0
        with pytest.raises(dfa.DfaError) as e:
            _lib._check(_lib.lib().dfa_mixture_sample(ctypes.byref(dfa.MixtureDesc(**bad)), FAKE, FAKE, FAKE, FAKE,
                                                      FAKE, FAKE, None, FAKE, 1 << 20, None))
        assert _lib.STATUS[e.value.status] == "DFA_ERR_SHAPE"
    need = dfa.dfa_mixture_workspace_size(d)

    def call(**kw):
        p = dict(l1=FAKE, l2=FAKE, u=FAKE, tok=FAKE, gr=FAKE, al=FAKE, pm=None, ws=FAKE, nb=need)
        p.update(kw)
        with pytest.raises(dfa.DfaError) as e:
            _lib._check(_lib.lib().dfa_mixture_sample(ctypes.byref(d), p["l1"], p["l2"], p["u"], p["tok"], p["gr"],
                                                      p["al"], p["pm"], p["ws"], p["nb"], None))
        return _lib.STATUS[e.value.status]

    for name in ("l1", "l2", "u", "tok", "gr", "al"):
        assert call(**{name: None}, nb=0) == "DFA_ERR_NULL", name
    assert call(nb=need - 4) == "DFA_ERR_WORKSPACE"
    assert call(ws=None) == "DFA_ERR_WORKSPACE"
    for name in ("l1", "l2", "pm"):
        assert call(**{name: FAKE + 4}, nb=need - 4) == "DFA_ERR_ALIGNMENT", name
    assert call(ws=FAKE + 4) == "DFA_ERR_ALIGNMENT"


def moe_desc(**kw):
    d = dict(batch=32, hidden=4096, mlp=1024, num_experts=64, k1=4, k2=8, x_exact_bf16=1)
    d.update(kw)
    return dfa.MoeDesc(**d)


def test_moe_sizes_and_validation():
    d = moe_desc()
    # sel int32 [32][8] | g1 float [32][4] | g2 float [32][8], 16-byte aligned sections
    assert dfa.dfa_moe_routing_size(d) == 32 * 8 * 4 + 32 * 4 * 4 + 32 * 8 * 4
    assert dfa.dfa_moe_routing_size(moe_desc(batch=3, k1=1, k2=3)) == 48 + 16 + 48
    assert dfa.dfa_moe_workspace_size(d) == 4 * 32 * 8 * 2 * (1024 + 4096)
    # larger batches: the routing grows with the batch, the workspace holds one slice of 32 sequences
    assert dfa.dfa_moe_routing_size(moe_desc(batch=70)) == 70 * 8 * 4 + 70 * 4 * 4 + 70 * 8 * 4
    assert dfa.dfa_moe_workspace_size(moe_desc(batch=70)) == 4 * 32 * 8 * 2 * (1024 + 4096)
    assert dfa.dfa_moe_workspace_size(moe_desc(batch=5)) == 4 * 5 * 8 * 2 * (1024 + 4096)
    for bad in (dict(batch=0), dict(batch=65536), dict(hidden=4000), dict(mlp=64), dict(num_experts=0),
                dict(num_experts=1025), dict(k1=0), dict(k1=9), dict(k2=65), dict(num_experts=40, k2=33, k1=1)):
        bd = moe_desc(**bad)
        assert dfa.dfa_moe_routing_size(bd) == 0 and dfa.dfa_moe_workspace_size(bd) == 0, bad
        with pytest.raises(dfa.DfaError) as e:
            _lib._check(_lib.lib().dfa_moe_route(ctypes.byref(bd), FAKE, FAKE, FAKE, 1 << 20, None))
        assert _lib.STATUS[e.value.status] == "DFA_ERR_SHAPE", bad


def test_moe_call_errors():
    d = moe_desc()
    rb, wb = dfa.dfa_moe_routing_size(d), dfa.dfa_moe_workspace_size(d)

    def route(**kw):
        p = dict(r1=FAKE, r2=FAKE, rt=FAKE, nb=rb)
        p.update(kw)
        with pytest.raises(dfa.DfaError) as e:
            _lib._check(_lib.lib().dfa_moe_route(ctypes.byref(d), p["r1"], p["r2"], p["rt"], p["nb"], None))
        return _lib.STATUS[e.value.status]

    def ffn(**kw):
        p = dict(wg=FAKE, wu=FAKE, wd=FAKE, b=None, c=None, h1=FAKE, h2=FAKE, res1=None, res2=None, rt=FAKE,
                 o1=FAKE, o2=FAKE, ws=FAKE, nb=wb - 4)
        p.update(kw)
        with pytest.raises(dfa.DfaError) as e:
            _lib._check(_lib.lib().dfa_moe_ffn(ctypes.byref(d), p["wg"], p["wu"], p["wd"], p["b"], p["c"], p["h1"],
                                               p["h2"], p["res1"], p["res2"], p["rt"], p["o1"], p["o2"], p["ws"],
                                               p["nb"], None))
        return _lib.STATUS[e.value.status]

    for name in ("r1", "r2", "rt"):
        assert route(**{name: None}) == "DFA_ERR_NULL"
        assert route(**{name: FAKE + 4}) == "DFA_ERR_ALIGNMENT"
    assert route(nb=rb - 4) == "DFA_ERR_WORKSPACE"
    for name in ("wg", "wu", "wd", "h1", "h2", "rt", "o1", "o2"):
        assert ffn(**{name: None}) == "DFA_ERR_NULL", name
    for name in ("wg", "b", "c", "h2", "res1", "res2", "o2"):
        assert ffn(**{name: FAKE + 4}) == "DFA_ERR_ALIGNMENT", name
    assert ffn() == "DFA_ERR_WORKSPACE"
    assert ffn(ws=None, nb=wb) == "DFA_ERR_WORKSPACE"


def prefill_desc(**kw):
    d = dict(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, max_prompt_len=4096, block_size=16,
             max_blocks_per_seq=257, num_blocks=1028, scale=1 / math.sqrt(128))
    d.update(kw)
    return dfa.PrefillDesc(**d)


@pytest.mark.parametrize("change,status", [
    (dict(batch=0), "DFA_ERR_SHAPE"), (dict(num_q_heads=30), "DFA_ERR_SHAPE"),
    (dict(num_q_heads=24), "DFA_ERR_UNSUPPORTED"),  # 3 query heads per kv head
    (dict(num_q_heads=256), "DFA_ERR_UNSUPPORTED"),  # 32 per kv head
    (dict(head_dim=96), "DFA_ERR_UNSUPPORTED"), (dict(block_size=24), "DFA_ERR_SHAPE"),
    (dict(max_prompt_len=0), "DFA_ERR_SHAPE"), (dict(max_prompt_len=257 * 16 + 1), "DFA_ERR_SHAPE"),
    (dict(scale=0.0), "DFA_ERR_SHAPE"), (dict(scale=float("inf")), "DFA_ERR_SHAPE"),
    (dict(max_prompt_len=2048 * 16 + 16, max_blocks_per_seq=4096), "DFA_ERR_UNSUPPORTED"),  # over 2048 blocks
])
def test_prefill_validation(change, status):
    with pytest.raises(dfa.DfaError) as e:
        _lib._check(_lib.lib().dfa_prefill(ctypes.byref(prefill_desc(**change)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, None))
    assert _lib.STATUS[e.value.status] == status


def test_prefill_pointer_errors():
    names = ["q", "k", "v", "lens", "kc", "vc", "table", "o"]
    for i, name in enumerate(names):
        for bad, status in ((None, "DFA_ERR_NULL"), (FAKE + 4, "DFA_ERR_ALIGNMENT")):
            args = [FAKE] * 8
            args[i] = bad
            with pytest.raises(dfa.DfaError) as e:
                _lib._check(_lib.lib().dfa_prefill(ctypes.byref(prefill_desc()), *args, None))
            assert _lib.STATUS[e.value.status] == status, name


def test_stack_validation():
    layer = dfa.LayerDesc(batch=4, hidden=256, num_q_heads=4, num_kv_heads=2, head_dim=64, mlp=256, block_size=16,
                          max_blocks_per_seq=4, num_blocks=16, max_ctx_len=64, scale=0.125, x_exact_bf16=1)
    ok = dict(layer=layer, num_layers=2, rope=dfa.DFA_ROPE_HALF, rope_max_pos=64, rms_norm=1, rms_eps=1e-5)
    assert dfa.dfa_decode_stack_workspace_size(dfa.StackDesc(**ok)) == \
        dfa.dfa_decode_layer_workspace_size(layer) + 3 * 2 * 4 * 256 * 4
    for bad in (dict(num_layers=0), dict(rope=3), dict(rope_max_pos=63), dict(rms_norm=2), dict(rms_eps=-1.0)):
        assert dfa.dfa_decode_stack_workspace_size(dfa.StackDesc(**dict(ok, **bad))) == 0, bad
    # no rotary tables with rope set
    arr = (dfa.StackLayer * 2)()
    with pytest.raises(dfa.DfaError) as e:
        _lib._check(_lib.lib().dfa_decode_stack(ctypes.byref(dfa.StackDesc(**ok)), arr, None, None, FAKE, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, FAKE, 1 << 30, None))
    assert _lib.STATUS[e.value.status] == "DFA_ERR_NULL"
    # norm weights are read in 16-byte pieces: a misaligned one is refused before any launch
    for lay in arr:
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "a", "b", "c"):
            setattr(lay.w, name, FAKE)
        lay.norm_attn, lay.norm_mlp, lay.k_cache, lay.v_cache = FAKE, FAKE, FAKE, FAKE
    arr[1].norm_mlp = FAKE + 4
    with pytest.raises(dfa.DfaError) as e:
        _lib._check(_lib.lib().dfa_decode_stack(ctypes.byref(dfa.StackDesc(**ok)), arr, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, FAKE, 1 << 30, None))
    assert _lib.STATUS[e.value.status] == "DFA_ERR_ALIGNMENT"


def _call_noalloc(d, **ptrs):
    p = dict(q1=FAKE, q2=FAKE, a=FAKE, k=FAKE, v=FAKE, table=FAKE, ctx=FAKE, o1=FAKE, o2=FAKE)
    p.update(ptrs)
    st = _lib.lib().dfa_decode_attn_noalloc(ctypes.byref(d), p["q1"], p["q2"], p["a"], p["k"], p["v"], p["table"],
                                            p["ctx"], p["o1"], p["o2"], None)
    _lib._check(st)


def test_noalloc_validates_like_decode_attn_and_checks_its_scratch_limit():
    # an invalid descriptor: the same status as dfa_decode_attn, nothing reaches the GPU
    with pytest.raises(dfa.DfaError) as e:
        _call_noalloc(c2_desc(num_flows=3))
    assert _lib.STATUS[e.value.status] == "DFA_ERR_SHAPE"
    with pytest.raises(dfa.DfaError) as e:
        _call_noalloc(c2_desc(split_len=512), q1=None)
    assert _lib.STATUS[e.value.status] == "DFA_ERR_NULL"
    # records beyond the fixed 8 MiB scratch: refused on the host before any device call
    d = c2_desc(batch=64, num_q_heads=64, block_size=4096, max_blocks_per_seq=1, num_blocks=64, split_len=256)
    assert dfa.dfa_decode_attn_workspace_size(d) > 8 << 20
    with pytest.raises(dfa.DfaError) as e:
        _call_noalloc(d)
    assert _lib.STATUS[e.value.status] == "DFA_ERR_WORKSPACE"
    assert "scratch" in _lib.lib().dfa_last_error().decode()


def test_table_check_validation():
    """dfa_check_kv_table: the descriptor's checks, then its own (pointers, alignment, ctx_add), all on the
    host before any device call."""
    call = lambda d, table=FAKE, ctx=FAKE, add=0, flags=FAKE: _lib._check(
        _lib.lib().dfa_check_kv_table(ctypes.byref(d), table, ctx, add, flags, None))
    for kw, args, status in ((dict(num_flows=3), {}, "DFA_ERR_SHAPE"),
                             ({}, dict(flags=None), "DFA_ERR_NULL"),
                             ({}, dict(table=None), "DFA_ERR_NULL"),
                             ({}, dict(ctx=FAKE + 4), "DFA_ERR_ALIGNMENT"),
                             ({}, dict(add=2), "DFA_ERR_SHAPE"),
                             ({}, dict(add=-1), "DFA_ERR_SHAPE")):
        with pytest.raises(dfa.DfaError) as e:
            call(c2_desc(**kw), **args)
        assert _lib.STATUS[e.value.status] == status, (kw, args)


def test_output_head_plans_and_validation():
    """dfa_output_head: its workspace (GEMV partials when the plan splits k, then the mixture's chunk
    records); every error on the host."""
    head = lambda **kw: dfa.HeadDesc(**{**dict(batch=32, vocab=32000, hidden=4096, x_exact_bf16=1), **kw})
    up = lambda x: (x + 255) // 256 * 256
    # 32000 tokens: the one-launch mixture (8 chunk records of 4096 tokens per sequence)
    assert dfa.dfa_output_head_workspace_size(head()) == up(32 * 8 * 8 * 4) + up(32 * 8 * 16)
    # 40960 tokens: 10 chunks
    assert dfa.dfa_output_head_workspace_size(head(vocab=40960, hidden=2048)) == up(32 * 10 * 8 * 4) + \
        up(32 * 10 * 16)
    # 4160 x 512: 65 row groups of 64 split k (4 ranges of 128 columns): partials, then chunk records
    gd = dfa.GemvDesc(batch=3, n=4160, k=512, num_flows=2, epilogue=0, x_exact_bf16=1, k_split=0, rows_per_wg=0)
    g = dfa.dfa_dual_gemv_workspace_size(gd)
    assert g > 0
    assert dfa.dfa_output_head_workspace_size(head(batch=3, vocab=4160, hidden=512)) == up(g) + up(3 * 2 * 8 * 4) + \
        up(3 * 2 * 16)
    for bad in (dict(batch=0), dict(batch=65536), dict(vocab=32001), dict(vocab=0), dict(vocab=(1 << 20) + 64),
                dict(hidden=100)):
        assert dfa.dfa_output_head_workspace_size(head(**bad)) == 0, bad
    call = lambda d, **kw: _lib._check(_lib.lib().dfa_output_head(
        ctypes.byref(d), *[kw.get(n, FAKE) for n in ("w", "h1", "h2", "u", "l1", "l2", "tok", "gr", "al")],
        kw.get("pm"), kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None))
    for kw, status in ((dict(w=None), "DFA_ERR_NULL"), (dict(l2=None), "DFA_ERR_NULL"),
                       (dict(h1=FAKE + 4), "DFA_ERR_ALIGNMENT"), (dict(ws=None), "DFA_ERR_WORKSPACE"),
                       (dict(wsb=16), "DFA_ERR_WORKSPACE")):
        with pytest.raises(dfa.DfaError) as e:
            call(head(), **kw)
        assert _lib.STATUS[e.value.status] == status, kw
    with pytest.raises(dfa.DfaError) as e:
        call(head(vocab=100))
    assert _lib.STATUS[e.value.status] == "DFA_ERR_SHAPE"
