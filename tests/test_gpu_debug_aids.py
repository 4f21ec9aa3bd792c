"""Debug aids on the GPU: guard bands around every buffer a call writes, and the device-side check of
block-table entries (dfa_check_kv_table).

Guard bands: each output, workspace and cache buffer sits inside a larger allocation whose 16 KiB
before and after hold a NaN bit pattern (0x7FBADBAD) that no kernel writes; after the call both bands
must be intact, and the results must still match the oracle. Covered: decode attention (one split,
several splits, an empty sequence, the partials + combine path), the dual GEMV with and without split-K,
the whole layer step (outputs, workspace and the cache it appends to), mixture sampling on both
vocabulary paths, the MoE FFN and prefill (outputs and caches).

Table check: a valid paged table gives no flag; an entry out of [0, num_blocks) among the entries a
sequence reads, a length beyond max_ctx_len (also through ctx_add = 1) and a negative length are each
reported with the first offending sequence; entries past a sequence's length are not read and so not
reported; the clamped reads the attention kernels make of the same corrupt table stay inside the
cache (the guard bands around it are intact).
"""
import dataclasses

import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import assert_close, desc_for, oracle_attn, say
from oracle import formats as F
from oracle import layer as LY
from oracle import mixture as MX
from oracle import moe as MO
from oracle import prefill as PF
from workloads.device import to_device

pytestmark = pytest.mark.gpu

CANARY = 0x7FBADBAD
GUARD = 4096  # int32 words on each side


class Guarded:
    """A buffer of `shape` and `dtype` with guard bands of CANARY words before and after it."""

    def __init__(self, shape, dtype=torch.float32, fill=None, src=None):
        self.shape = tuple(shape)
        n = int(np.prod(self.shape)) if self.shape else 1
        esz = torch.empty((), dtype=dtype).element_size()
        self.words = max((n * esz + 3) // 4, 1)
        pad = (self.words + 3) // 4 * 4  # keeps the tail band 16-byte aligned
        self.raw = torch.full((2 * GUARD + pad,), CANARY, dtype=torch.int32, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.words].view(dtype)[:n].view(self.shape)
        if src is not None:
            self.t.copy_(src)
        elif fill is not None:
            self.t.fill_(fill)

    def intact(self):
        torch.cuda.synchronize()
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.words:]
        return bool((head == CANARY).all()) and bool((tail == CANARY).all())


def guard_like(x, fill=None):
    """A guarded device copy of tensor or array `x` (or a guarded buffer of its shape filled with `fill`)."""
    if not torch.is_tensor(x):
        x = to_device(np.ascontiguousarray(x))
    return Guarded(x.shape, x.dtype, src=None if fill is not None else x, fill=fill)


def assert_intact(**bufs):
    bad = [name for name, g in bufs.items() if not g.intact()]
    assert not bad, f"guard band overwritten next to: {', '.join(bad)}"


# ---------------------------------------------------------------- attention
ATTN = {
    "ragged": (W.C2.replace(batch=3, ctx_lens=(1000, 4096, 37), capacity=4096), 3101),
    "paged": (W.C3.replace(batch=6, ctx_range=None, ctx_lens=(1, 17, 33, 700, 1024, 513)), 3102),
    "empty": (W.AttnConfig("empty", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                           ctx_lens=(70, 0, 5), block_size=16, shuffle_blocks=True), 3103),
    "f32q_d64": (W.AttnConfig("f32q_d64", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64, dtype="bf16",
                              ctx_lens=(300, 1), q_dtype="f32"), 3104),
}


def check_attn_outputs(case, o1, o2, what):
    """Empty sequences give zero rows; the others match the oracle (which takes only non-empty contexts)."""
    empty = case.ctx_lens == 0
    assert np.all(o1[empty] == 0) and np.all(o2[empty] == 0), f"{what}: empty sequences"
    keep = ~empty
    ref = oracle_attn(dataclasses.replace(case, q1=case.q1[keep], q2=case.q2[keep], block_table=case.block_table[keep],
                                          ctx_lens=case.ctx_lens[keep]))
    assert_close(o1[keep], ref["o1"], what=f"{what} o1")
    assert_close(o2[keep], ref["o2"], what=f"{what} o2")


@pytest.mark.parametrize("split", [0, 32, 256])
@pytest.mark.parametrize("name", sorted(ATTN))
def test_attention_guard_bands(name, split):
    cfg, seed = ATTN[name]
    case = W.make_attn_case(cfg, seed)
    d = desc_for(case, 2, split)
    B, H, D = cfg.batch, cfg.num_q_heads, cfg.head_dim
    ins = {k: guard_like(getattr(case, k)) for k in ("q1", "q2", "a", "k_cache", "v_cache", "block_table",
                                                      "ctx_lens")}
    o1, o2 = Guarded((B, H, D), fill=float("nan")), Guarded((B, H, D), fill=float("nan"))
    ws_bytes = dfa.dfa_decode_attn_workspace_size(d)
    ws = Guarded((max(ws_bytes // 4, 1),), fill=float("nan"))
    say(f"case attention guard bands {name} split={split} ({dfa.dfa_decode_attn_num_splits(d)} split(s))")
    dfa.dfa_decode_attn(d, ins["q1"].t, ins["q2"].t, ins["a"].t, ins["k_cache"].t, ins["v_cache"].t,
                        ins["block_table"].t, ins["ctx_lens"].t, ws.t if ws_bytes else None, o1.t, o2.t)
    assert_intact(o1=o1, o2=o2, workspace=ws, **ins)
    check_attn_outputs(case, o1.t.cpu().numpy(), o2.t.cpu().numpy(), name)
    if ws_bytes:  # the two-pass path: records to the guarded workspace, then the combine
        p1, p2 = Guarded((B, H, D), fill=float("nan")), Guarded((B, H, D), fill=float("nan"))
        dfa.dfa_decode_attn_partials(d, ins["q1"].t, ins["q2"].t, ins["a"].t, ins["k_cache"].t, ins["v_cache"].t,
                                     ins["block_table"].t, ins["ctx_lens"].t, ws.t)
        dfa.dfa_combine(d, ws.t, p1.t, p2.t)
        assert_intact(o1=p1, o2=p2, workspace=ws)
        assert torch.equal(p1.t, o1.t) and torch.equal(p2.t, o2.t)


# ---------------------------------------------------------------- GEMV
def _pack(w_bits):
    n, k = w_bits.shape
    w = to_device(w_bits)
    wt = torch.empty_like(w)
    dfa.dfa_pack_weight(w, wt, n, k)
    return wt


@pytest.mark.parametrize("batch,k_split,rows", [(17, 0, 0), (32, 3, 0), (5, 2, 128)])
def test_gemv_guard_bands(batch, k_split, rows):
    rng = np.random.default_rng(batch + 7 * k_split)
    n, k = 256, 384
    x1, x2 = rng.standard_normal((2, batch, k)).astype(np.float32)
    r1, r2 = rng.standard_normal((2, batch, n)).astype(np.float32)
    w = W.f32_to_bf16_bits(rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02))
    d = dfa.GemvDesc(batch=batch, n=n, k=k, num_flows=2, epilogue=dfa.DFA_EPI_RESIDUAL, x_exact_bf16=0,
                     k_split=k_split, rows_per_wg=rows)
    ws_bytes = dfa.dfa_dual_gemv_workspace_size(d)
    ws = Guarded((max(ws_bytes // 4, 1),), fill=float("nan"))
    wt = guard_like(_pack(w))
    g = {name: guard_like(v) for name, v in (("x1", x1), ("x2", x2), ("res1", r1), ("res2", r2))}
    y1, y2 = Guarded((batch, n), fill=float("nan")), Guarded((batch, n), fill=float("nan"))
    say(f"case gemv guard bands batch={batch} k_split={k_split} rows={rows}")
    dfa.dfa_dual_gemv(d, wt.t, None, g["x1"].t, g["x2"].t, None, g["res1"].t, g["res2"].t, y1.t, y2.t, None,
                      ws.t if ws_bytes else None)
    assert_intact(y1=y1, y2=y2, workspace=ws, w=wt, **g)
    assert_close(y1.t.cpu().numpy(), r1 + LY.linear(x1.astype(np.float64), w), what="y1")
    assert_close(y2.t.cpu().numpy(), r2 + LY.linear(x2.astype(np.float64), w), what="y2")


# ---------------------------------------------------------------- layer step
def test_layer_guard_bands():
    cfg = W.C5.replace(batch=5, hidden=256, num_q_heads=4, num_kv_heads=1, head_dim=128, mlp=384, ctx=300,
                       block_size=16, shuffle_blocks=True)
    case = W.make_layer_case(cfg, 3201)
    packed = {name: _pack(case.w[name]) for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}
    ins = {name: guard_like(getattr(case, name)) for name in ("x1", "x2", "a", "b", "c", "block_table",
                                                               "ctx_lens")}
    k, v = guard_like(case.k_cache), guard_like(case.v_cache)
    desc = dfa.LayerDesc(batch=cfg.batch, hidden=cfg.hidden, num_q_heads=cfg.num_q_heads,
                         num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, mlp=cfg.mlp,
                         block_size=case.block_size, max_blocks_per_seq=case.max_blocks_per_seq,
                         num_blocks=case.k_cache.shape[0], max_ctx_len=int(case.ctx_lens.max()) + 1,
                         scale=cfg.scale, x_exact_bf16=1)
    wts = dfa.layer_weights(packed["wq"], packed["wk"], packed["wv"], packed["wo"], packed["wg"], packed["wu"],
                            packed["wd"], ins["a"].t, ins["b"].t, ins["c"].t)
    ws = Guarded((dfa.dfa_decode_layer_workspace_size(desc) // 4,), fill=float("nan"))
    out1 = Guarded(case.x1.shape, fill=float("nan"))
    out2 = Guarded(case.x1.shape, fill=float("nan"))
    say("case layer guard bands")
    dfa.dfa_decode_layer(desc, wts, ins["x1"].t, ins["x2"].t, k.t, v.t, ins["block_table"].t, ins["ctx_lens"].t,
                         out1.t, out2.t, ws.t)
    assert_intact(out1=out1, out2=out2, workspace=ws, k_cache=k, v_cache=v, **ins)
    ref = LY.dual_flow_layer(case.x1, case.x2, case.w, case.a, case.b, case.c, case.k_cache, case.v_cache,
                             case.block_table, case.ctx_lens, num_q_heads=cfg.num_q_heads,
                             num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, scale=cfg.scale,
                             block_size=case.block_size)
    assert_close(out1.t.cpu().numpy(), ref["out1"], what="layer out1")
    assert_close(out2.t.cpu().numpy(), ref["out2"], what="layer out2")


# ---------------------------------------------------------------- mixture sampling
@pytest.mark.parametrize("vocab", [32000, 40000])
def test_mixture_guard_bands(vocab):
    rng = np.random.default_rng(vocab)
    batch = 3
    l1, l2 = (rng.standard_normal((2, batch, vocab)) * 3).astype(np.float32)
    u = rng.random(batch).astype(np.float32)
    d = dfa.MixtureDesc(batch=batch, vocab=vocab)
    g1, g2, gu = guard_like(l1), guard_like(l2), guard_like(u)
    tok = Guarded((batch,), torch.int32, fill=-7)
    gr = Guarded((batch,), torch.int32, fill=-7)
    al = Guarded((batch,), fill=float("nan"))
    pm = Guarded((batch, vocab), fill=float("nan"))
    ws = Guarded((dfa.dfa_mixture_workspace_size(d) // 4,), fill=float("nan"))
    say(f"case mixture guard bands vocab={vocab}")
    dfa.dfa_mixture_sample(d, g1.t, g2.t, gu.t, tok.t, gr.t, al.t, pm.t, ws.t)
    assert_intact(token=tok, greedy=gr, alpha=al, p_mix=pm, workspace=ws, logits1=g1, logits2=g2, u=gu)
    ref = MX.mixture(l1, l2)
    assert_close(pm.t.cpu().numpy(), ref["p_mix"], what="p_mix")
    assert np.max(np.abs(al.t.cpu().numpy() - ref["alpha"])) <= 5e-5


# ---------------------------------------------------------------- MoE FFN
def test_moe_guard_bands():
    cfg = W.MoeConfig("moe_small", batch=5, hidden=256, mlp=128, experts=9, k1=2, k2=4)
    case = W.make_moe_case(cfg, 3301)
    d = dfa.MoeDesc(batch=cfg.batch, hidden=cfg.hidden, mlp=cfg.mlp, num_experts=cfg.experts, k1=cfg.k1,
                    k2=cfg.k2, x_exact_bf16=1)
    r1, r2 = _router_logits(case)
    rt = MO.route(r1, r2, cfg.k1, cfg.k2)
    routing = Guarded((dfa.dfa_moe_routing_size(d) // 4,), torch.int32, fill=0)
    gr1, gr2 = guard_like(r1), guard_like(r2)
    say("case moe guard bands: route")
    dfa.dfa_moe_route(d, gr1.t, gr2.t, routing.t)
    assert_intact(routing=routing, r1=gr1, r2=gr2)
    experts = {name: _pack_experts(getattr(case, name)) for name in ("wg", "wu", "wd")}
    ins = {name: guard_like(np.ascontiguousarray(getattr(case, name), dtype=np.float32))
           for name in ("h1", "h2", "res1", "res2")}
    gb, gc = guard_like(case.b), guard_like(case.c)
    out1 = Guarded((cfg.batch, cfg.hidden), fill=float("nan"))
    out2 = Guarded((cfg.batch, cfg.hidden), fill=float("nan"))
    ws = Guarded((dfa.dfa_moe_workspace_size(d) // 4,), fill=float("nan"))
    say("case moe guard bands: ffn")
    dfa.dfa_moe_ffn(d, experts["wg"].t, experts["wu"].t, experts["wd"].t, gb.t, gc.t, ins["h1"].t, ins["h2"].t,
                    ins["res1"].t, ins["res2"].t, routing.t, out1.t, out2.t, ws.t)
    assert_intact(out1=out1, out2=out2, workspace=ws, routing=routing, b=gb, c=gc, **ins, **experts)
    ref = MO.moe_ffn(case.h1, case.h2, case.res1, case.res2, case.wg, case.wu, case.wd, case.b, case.c, rt["sel"],
                     rt["g1"], rt["g2"])
    assert_close(out1.t.cpu().numpy(), ref["out1"], what="moe out1")
    assert_close(out2.t.cpu().numpy(), ref["out2"], what="moe out2")


def _router_logits(case):
    wr = F.to_f64(case.wr, "bf16")
    return (case.h1 @ wr.T).astype(np.float32), (case.h2 @ wr.T).astype(np.float32)


def _pack_experts(w_bits):
    ne, n, k = w_bits.shape
    src = to_device(np.ascontiguousarray(w_bits))
    dst = guard_like(src, fill=0)
    for e in range(ne):
        dfa.dfa_pack_weight(src[e], dst.t[e], n, k)
    return dst


# ---------------------------------------------------------------- prefill
def test_prefill_guard_bands():
    cfg = W.PrefillConfig("g8", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=64, lens=(0, 95, 64),
                          block_size=64)
    case = W.make_prefill_case(cfg, 3401)
    ins = {name: guard_like(getattr(case, name)) for name in ("q", "k", "v", "lens", "block_table")}
    kc, vc = guard_like(case.k_cache), guard_like(case.v_cache)
    o = Guarded(case.q.shape, fill=-12345.0)
    d = dfa.PrefillDesc(batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                        head_dim=cfg.head_dim, max_prompt_len=case.q.shape[1], block_size=case.block_size,
                        max_blocks_per_seq=case.max_blocks_per_seq, num_blocks=case.k_cache.shape[0],
                        scale=cfg.scale)
    say("case prefill guard bands")
    dfa.dfa_prefill(d, ins["q"].t, ins["k"].t, ins["v"].t, ins["lens"].t, kc.t, vc.t, ins["block_table"].t, o.t)
    assert_intact(o=o, k_cache=kc, v_cache=vc, **ins)
    ref = PF.causal_attention(case.q, case.k, case.v, case.lens, num_kv_heads=cfg.num_kv_heads, scale=cfg.scale)
    got = o.t.cpu().numpy()
    for b in range(cfg.batch):
        n = int(case.lens[b])
        if n:
            assert_close(got[b, :n], ref[b, :n], what=f"prefill prompt {b}")


# ---------------------------------------------------------------- table check
def check_table(d, table, ctx, ctx_add=0):
    flags = Guarded((2,), torch.int32, fill=-7)
    dfa.dfa_check_kv_table(d, table, ctx, flags.t, ctx_add=ctx_add)
    assert_intact(flags=flags)
    bits, first = (int(x) & 0xFFFFFFFF for x in flags.t.cpu().numpy())
    return bits, (None if first == 0xFFFFFFFF else first)


def test_table_check_flags():
    cfg, seed = ATTN["paged"]
    case = W.make_attn_case(cfg, seed)
    d = desc_for(case, 2, 0)
    table, ctx = to_device(case.block_table), to_device(case.ctx_lens)
    nb = case.k_cache.shape[0]
    say("case table check: valid table")
    assert check_table(d, table, ctx) == (0, None)
    # the layer step reads one more position: fine while that stays within max_ctx_len
    assert check_table(d, table, ctx - 1, ctx_add=1) == (0, None)
    # ... and reported when it does not (the length read is clamped to max_ctx_len, whose entries are valid)
    assert check_table(d, table, ctx, ctx_add=1) == (dfa.DFA_TABLE_BAD_LEN, int(np.argmax(case.ctx_lens)))
    # entries past a sequence's length are never read: not reported
    lens = case.ctx_lens
    b_short = int(np.argmin(lens))
    used = -(-int(lens[b_short]) // case.block_size)
    assert used < case.max_blocks_per_seq
    t2 = table.clone()
    t2[b_short, used:] = -1
    assert check_table(d, t2, ctx) == (0, None)
    # a bad entry the kernels read: reported with its sequence
    for b, j, val in ((4, 0, nb), (3, used_of(case, 3) - 1, -1), (5, 1, nb + 1000)):
        t3 = table.clone()
        t3[b, j] = val
        say(f"case table check: entry ({b}, {j}) = {val}")
        assert check_table(d, t3, ctx) == (dfa.DFA_TABLE_BAD_BLOCK, b)
    # two bad rows: the first is named
    t4 = table.clone()
    t4[5, 0] = nb
    t4[2, 0] = -3
    assert check_table(d, t4, ctx) == (dfa.DFA_TABLE_BAD_BLOCK, 2)
    # lengths: beyond max_ctx_len, negative; an empty sequence is valid
    c2 = ctx.clone()
    c2[1] = case.max_ctx_len + 1
    # read as max_ctx_len positions: the row's unused entries (-1) past its true length are then read too
    both = dfa.DFA_TABLE_BAD_LEN | dfa.DFA_TABLE_BAD_BLOCK
    assert check_table(d, table, c2) == (both, 1)
    c3 = ctx.clone()
    c3[3] = -2
    assert check_table(d, table, c3) == (dfa.DFA_TABLE_BAD_LEN, 3)
    c4 = ctx.clone()
    c4[0] = 0
    assert check_table(d, table, c4) == (0, None)
    # both kinds at once
    t5 = table.clone()
    t5[4, 0] = nb
    assert check_table(d, t5, c2) == (both, 1)


def used_of(case, b):
    return -(-int(case.ctx_lens[b]) // case.block_size)


def test_corrupt_table_reads_stay_inside_the_cache():
    """The attention kernels clamp what the check reports: with out-of-range entries and lengths the
    call still reads and writes only its own buffers."""
    cfg, seed = ATTN["paged"]
    case = W.make_attn_case(cfg, seed)
    d = desc_for(case, 2, 64)
    ins = {k: guard_like(getattr(case, k)) for k in ("q1", "q2", "a", "k_cache", "v_cache")}
    table = case.block_table.copy()
    table[4, 0] = case.k_cache.shape[0] + 5
    table[3, 1] = -100
    lens = case.ctx_lens.copy()
    lens[1] = case.max_ctx_len + 50
    gt, gl = guard_like(table), guard_like(lens)
    assert check_table(d, gt.t, gl.t) == (dfa.DFA_TABLE_BAD_LEN | dfa.DFA_TABLE_BAD_BLOCK, 1)
    B, H, D = cfg.batch, cfg.num_q_heads, cfg.head_dim
    o1, o2 = Guarded((B, H, D), fill=float("nan")), Guarded((B, H, D), fill=float("nan"))
    ws = Guarded((dfa.dfa_decode_attn_workspace_size(d) // 4,), fill=float("nan"))
    say("case corrupt table: attention on clamped reads")
    dfa.dfa_decode_attn(d, ins["q1"].t, ins["q2"].t, ins["a"].t, ins["k_cache"].t, ins["v_cache"].t, gt.t, gl.t,
                        ws.t, o1.t, o2.t)
    assert_intact(o1=o1, o2=o2, workspace=ws, table=gt, ctx_lens=gl, **ins)
    # sequences the corruption does not touch are unchanged
    ref = oracle_attn(case)
    ok = [0, 2, 5]
    assert_close(o1.t.cpu().numpy()[ok], ref["o1"][ok], what="untouched sequences o1")
    assert_close(o2.t.cpu().numpy()[ok], ref["o2"][ok], what="untouched sequences o2")
