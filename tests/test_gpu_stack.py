"""GPU parity of dfa_decode_stack (layers chained, RMSNorm, rotary embeddings) with oracle.stack, and its
capture in a HIP graph.

Bars: outputs within the row-normalised 2e-3 of the other GPU tests; every layer's cache differs from
the oracle's only at the appended slots, each appended value by at most one bf16 ulp or 1e-5 of the
largest appended magnitude of that layer (rotated components a cos - b sin can cancel to values far
below their row's scale, where the float32 projection's error, ~1e-6 of the scale, spans many ulps
of the small result). Invariants: the primary flow's outputs and every cache are bit for bit
independent of the auxiliary input; with neither option the stack equals consecutive dfa_decode_layer
calls bit for bit. A graph captured around one stack step replays it bit for bit, three times, with
eager work between the replays.
"""
import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import assert_close, say
from oracle import stack as ST
from workloads.device import to_device

pytestmark = pytest.mark.gpu

SMALL = W.C5.replace(batch=5, hidden=256, num_q_heads=4, num_kv_heads=2, head_dim=64, mlp=256, ctx=40, block_size=16,
                     shuffle_blocks=True, capacity=0)
WIDE = W.C5.replace(batch=8, hidden=1024, num_q_heads=8, num_kv_heads=2, head_dim=128, mlp=2048, ctx=300,
                    block_size=16, shuffle_blocks=True, capacity=0)
# 12288 MLP rows: the SwiGLU GEMV runs unsplit, its epilogue in the GEMV kernel (smaller MLPs split k and
# finish in the reduction); 40 sequences: GEMV slices of 32 and 8
TALL = W.C5.replace(batch=40, hidden=256, num_q_heads=4, num_kv_heads=2, head_dim=64, mlp=12288, ctx=40, block_size=16,
                    shuffle_blocks=True, capacity=0)
ROPE = {"none": dfa.DFA_ROPE_NONE, "half": dfa.DFA_ROPE_HALF, "interleaved": dfa.DFA_ROPE_INTERLEAVED}


def pack(w_bits):
    n, k = w_bits.shape
    w = to_device(w_bits)
    wt = torch.empty_like(w)
    dfa.dfa_pack_weight(w, wt, n, k)
    return wt


class Stack:
    """A stack case on the GPU: packed weights, norms, caches and tables."""

    def __init__(self, sc):
        self.sc = sc
        cfg = sc.cfg
        lc = cfg.layer
        self.entries = []
        for li, w in enumerate(sc.layers):
            lw = dfa.layer_weights(pack(w["wq"]), pack(w["wk"]), pack(w["wv"]), pack(w["wo"]), pack(w["wg"]),
                                   pack(w["wu"]), pack(w["wd"]), to_device(w["a"]), to_device(w["b"]), to_device(w["c"]))
            self.entries.append((lw, to_device(w["n_attn"].astype(np.float32)), to_device(w["n_mlp"].astype(np.float32)),
                                 to_device(sc.k_caches[li]), to_device(sc.v_caches[li])))
        self.layers = dfa.stack_layers(self.entries)
        self.desc = dfa.StackDesc(
            layer=dfa.LayerDesc(batch=lc.batch, hidden=lc.hidden, num_q_heads=lc.num_q_heads,
                                num_kv_heads=lc.num_kv_heads, head_dim=lc.head_dim, mlp=lc.mlp,
                                block_size=sc.block_size, max_blocks_per_seq=sc.max_blocks_per_seq,
                                num_blocks=sc.k_caches[0].shape[0], max_ctx_len=lc.ctx + 1, scale=lc.scale,
                                x_exact_bf16=1),
            num_layers=cfg.layers, rope=ROPE[cfg.rope], rope_max_pos=sc.cos.shape[0], rms_norm=int(cfg.rms),
            rms_eps=cfg.eps)
        self.cos, self.sin = to_device(sc.cos), to_device(sc.sin)
        self.x1, self.x2 = to_device(sc.x1), to_device(sc.x2)
        self.table, self.ctx = to_device(sc.block_table), to_device(sc.ctx_lens)
        self.ws = torch.empty(dfa.dfa_decode_stack_workspace_size(self.desc) // 4 + 64, device="cuda")
        self.out1 = torch.full(tuple(sc.x1.shape), float("nan"), device="cuda")
        self.out2 = torch.full_like(self.out1, float("nan"))

    def step(self, x2=None):
        dfa.dfa_decode_stack(self.desc, self.layers, self.cos, self.sin, self.x1, self.x2 if x2 is None else x2,
                             self.table, self.ctx, self.out1, self.out2, self.ws)

    def caches(self):
        return [(e[3].cpu().numpy().view(np.uint16), e[4].cpu().numpy().view(np.uint16)) for e in self.entries]


def bf16_ulp_diff(a_bits, b_bits):
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def oracle(sc):
    lc = sc.cfg.layer
    return ST.stack_step(sc.x1, sc.x2, sc.layers, sc.k_caches, sc.v_caches, sc.block_table, sc.ctx_lens,
                         num_q_heads=lc.num_q_heads, num_kv_heads=lc.num_kv_heads, head_dim=lc.head_dim,
                         scale=lc.scale, block_size=sc.block_size, rope_style=sc.cfg.rope, cos=sc.cos, sin=sc.sin,
                         rms=sc.cfg.rms, eps=sc.cfg.eps)


CASES = [("half", True, SMALL, 3), ("interleaved", True, SMALL, 3), ("half", False, SMALL, 2),
         ("none", True, SMALL, 2), ("half", True, WIDE, 2), ("interleaved", False, WIDE, 2),
         ("half", True, TALL, 2)]


@pytest.mark.parametrize("rope,rms,layer,layers", CASES,
                         ids=[f"{r}-{'rms' if n else 'plain'}-d{c.head_dim}-b{c.batch}-m{c.mlp}-L{l}"
                              for r, n, c, l in CASES])
def test_stack_matches_oracle(rope, rms, layer, layers):
    sc = W.make_stack_case(W.StackConfig("t", layer, layers=layers, rope=rope, rms=rms), 71)
    say(f"case stack rope {rope} rms {rms} layers {layers} head_dim {layer.head_dim}")
    g = Stack(sc)
    g.step()
    torch.cuda.synchronize()
    ref = oracle(sc)
    assert_close(g.out1.cpu().numpy(), ref["out1"], what="stack out1")
    assert_close(g.out2.cpu().numpy(), ref["out2"], what="stack out2")
    n_app = layer.batch * layer.num_kv_heads * layer.head_dim
    for li, ((k, v), (rk, rv)) in enumerate(zip(g.caches(), ref["caches"])):
        for got, want, base in ((k, rk, sc.k_caches[li]), (v, rv, sc.v_caches[li])):
            diff = got != want
            assert diff.sum() <= n_app and (got != base).sum() <= n_app, f"layer {li}"
            if diff.any():
                changed = want != base
                scale = np.abs(W.bf16_bits_to_f32(want[changed])).max()
                gd, wd = W.bf16_bits_to_f32(got[diff]), W.bf16_bits_to_f32(want[diff])
                ok = (bf16_ulp_diff(got[diff], want[diff]) <= 1) | (np.abs(gd - wd) <= 1e-5 * scale)
                assert np.all(ok), f"layer {li}: {gd[~ok]} vs {wd[~ok]} (scale {scale})"


def test_stack_primary_independence_and_plain_layers():
    sc = W.make_stack_case(W.StackConfig("t", SMALL, layers=3, rope="half", rms=True), 72)
    say("case stack: primary independence")
    g = Stack(sc)
    g.step()
    o1, c = g.out1.cpu().numpy(), g.caches()
    g2 = Stack(sc)
    g2.step(x2=to_device(W.bf16_bits_to_f32(W.f32_to_bf16_bits(sc.x2 * -2.0))))
    assert np.array_equal(g2.out1.cpu().numpy(), o1)
    for (k0, v0), (k1, v1) in zip(c, g2.caches()):
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    # neither option: the stack is consecutive dfa_decode_layer calls, bit for bit
    plain = W.make_stack_case(W.StackConfig("p", SMALL, layers=2, rope="none", rms=False), 73)
    gp = Stack(plain)
    gp.step()
    d = gp.desc.layer
    ws = torch.empty(dfa.dfa_decode_layer_workspace_size(d) // 4 + 64, device="cuda")
    x1, x2 = to_device(plain.x1), to_device(plain.x2)
    for li in range(2):
        lw, _, _, _, _ = gp.entries[li]
        k, v = to_device(plain.k_caches[li]), to_device(plain.v_caches[li])
        y1, y2 = torch.empty_like(x1), torch.empty_like(x2)
        dl = dfa.LayerDesc.from_buffer_copy(d)
        dl.x_exact_bf16 = 1 if li == 0 else 0  # a later layer's input is a float32 output
        dfa.dfa_decode_layer(dl, lw, x1, x2, k, v, gp.table, gp.ctx, y1, y2, ws)
        x1, x2 = y1, y2
    torch.cuda.synchronize()
    assert np.array_equal(x1.cpu().numpy(), gp.out1.cpu().numpy())
    assert np.array_equal(x2.cpu().numpy(), gp.out2.cpu().numpy())


def test_stack_graph_replays():
    sc = W.make_stack_case(W.StackConfig("g", SMALL, layers=3, rope="interleaved", rms=True), 74)
    say("case stack: HIP graph capture and replay")
    g = Stack(sc)
    g.step()
    torch.cuda.synchronize()
    eager1, eager2, eager_c = g.out1.cpu().numpy(), g.out2.cpu().numpy(), g.caches()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        g.step()
    for rep in range(3):
        g.out1.fill_(float("nan"))
        g.out2.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g.out1.cpu().numpy(), eager1), f"replay {rep}"
        assert np.array_equal(g.out2.cpu().numpy(), eager2), f"replay {rep}"
        for (k0, v0), (k1, v1) in zip(eager_c, g.caches()):
            assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
        del scratch
