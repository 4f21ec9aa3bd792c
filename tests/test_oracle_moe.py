"""Pins of oracle.moe: brute force, library routines, the dense layer as the one-expert case,
invariants, and planted mistakes.

The reading pinned (oracle/moe.py): experts ranked by the primary's router logits (ties to the
smaller index); the primary takes the first k1, the auxiliary flow replays the first k2 of the
same ranking; each flow mixes its experts with a softmax of its own router logits over its set;
b couples the SwiGLU intermediate where the primary ran the expert; c couples the MoE output.
"""
import math
import struct

import numpy as np
import pytest
import scipy.special

import workloads as W
from oracle import formats as F
from oracle import layer as LY
from oracle import moe as MO

TINY = W.MoeConfig("tiny", batch=3, hidden=8, mlp=6, experts=5, k1=2, k2=3, w_std=0.5)


def bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def brute_route(r1, r2, k1, k2):
    out = []
    for row1, row2 in zip(r1.tolist(), r2.tolist()):
        order = sorted(range(len(row1)), key=lambda e: (-row1[e], e))[:k2]
        def soft(vals):
            m = max(vals)
            ex = [math.exp(v - m) for v in vals]
            t = math.fsum(ex)
            return [x / t for x in ex]
        out.append((order, soft([row1[e] for e in order[:k1]]), soft([row2[e] for e in order])))
    return out


def brute_ffn(case, sel, g1, g2, b=True, c=True):
    """Scalar loops: own bf16 decoding, math.fsum dot products, math.exp silu."""
    cfg = case.cfg
    def matvec(w_bits, x):
        return [math.fsum(bf16(w_bits[i, j]) * x[j] for j in range(len(x))) for i in range(w_bits.shape[0])]
    def swiglu(e, x):
        a = matvec(case.wg[e], x)
        u = matvec(case.wu[e], x)
        return [ai / (1.0 + math.exp(-ai)) * ui for ai, ui in zip(a, u)]
    outs = []
    for s in range(cfg.batch):
        x1, x2 = case.h1[s].tolist(), case.h2[s].tolist()
        m1 = [0.0] * cfg.hidden
        m2 = [0.0] * cfg.hidden
        for slot, e in enumerate(sel[s]):
            z2 = swiglu(e, x2)
            if slot < len(g1[s]):
                z1 = swiglu(e, x1)
                y1 = matvec(case.wd[e], z1)
                m1 = [m + g1[s][slot] * y for m, y in zip(m1, y1)]
                if b:
                    z2 = [zz + float(bb) * z for zz, bb, z in zip(z2, case.b.tolist(), z1)]
            y2 = matvec(case.wd[e], z2)
            m2 = [m + g2[s][slot] * y for m, y in zip(m2, y2)]
        o1 = [float(r) + m for r, m in zip(case.res1[s].tolist(), m1)]
        o2 = [float(r) + m + (float(cc) * mm if c else 0.0)
              for r, m, cc, mm in zip(case.res2[s].tolist(), m2, case.c.tolist(), m1)]
        outs.append((o1, o2))
    return outs


def router_logits(case):
    wr = F.to_f64(case.wr, "bf16")
    return case.h1 @ wr.T, case.h2 @ wr.T


def tiny_case(seed=3, cfg=TINY):
    case = W.make_moe_case(cfg, seed)
    r1, r2 = router_logits(case)
    return case, r1, r2


def run_ffn(case, rt, **over):
    args = dict(h1=case.h1, h2=case.h2, res1=case.res1, res2=case.res2, wg=case.wg, wu=case.wu, wd=case.wd,
                b=case.b, c=case.c, sel=rt["sel"], g1=rt["g1"], g2=rt["g2"])
    args.update(over)
    return MO.moe_ffn(**args)


def test_route_brute_force_with_ties():
    rng = np.random.default_rng(1)
    r1 = rng.integers(-3, 3, size=(6, 9)).astype(np.float64)  # many ties
    r2 = rng.standard_normal((6, 9))
    got = MO.route(r1, r2, 3, 5)
    for s, (order, g1, g2) in enumerate(brute_route(r1, r2, 3, 5)):
        assert got["sel"][s].tolist() == order
        assert np.max(np.abs(got["g1"][s] - g1)) <= 1e-15 and np.max(np.abs(got["g2"][s] - g2)) <= 1e-15


def test_route_matches_library_routines():
    rng = np.random.default_rng(2)
    r1, r2 = rng.standard_normal((8, 64)), rng.standard_normal((8, 64))
    got = MO.route(r1, r2, 4, 8)
    top = np.argpartition(-r1, 8, axis=-1)[:, :8]
    for s in range(8):
        assert set(got["sel"][s].tolist()) == set(top[s].tolist())
        assert np.all(np.diff(r1[s, got["sel"][s]]) <= 0)  # ranking order
        assert np.allclose(got["g1"][s], scipy.special.softmax(r1[s, got["sel"][s, :4]]), rtol=0, atol=1e-15)
        assert np.allclose(got["g2"][s], scipy.special.softmax(r2[s, got["sel"][s]]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", [3, 4])
def test_ffn_brute_force(seed):
    case, r1, r2 = tiny_case(seed)
    rt = MO.route(r1, r2, TINY.k1, TINY.k2)
    got = run_ffn(case, rt)
    ref = brute_ffn(case, rt["sel"].tolist(), rt["g1"].tolist(), rt["g2"].tolist())
    for s, (o1, o2) in enumerate(ref):
        assert np.max(np.abs(got["out1"][s] - o1)) <= 1e-12
        assert np.max(np.abs(got["out2"][s] - o2)) <= 1e-12


def test_single_expert_is_the_dense_layer_mlp():
    """One expert with both fan-outs 1: gates are 1 and the MoE FFN is the dense layer's MLP stage."""
    cfg = W.C5.replace(batch=2, hidden=16, num_q_heads=2, num_kv_heads=1, head_dim=8, mlp=24, ctx=20,
                       block_size=16, shuffle_blocks=True)
    lc = W.make_layer_case(cfg, 31)
    r = LY.dual_flow_layer(lc.x1, lc.x2, lc.w, lc.a, lc.b, lc.c, lc.k_cache, lc.v_cache, lc.block_table,
                           lc.ctx_lens, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                           head_dim=cfg.head_dim, scale=cfg.scale, block_size=lc.block_size)
    rt = MO.route(np.zeros((2, 1)), np.zeros((2, 1)), 1, 1)
    got = MO.moe_ffn(r["h1"], r["h2"], r["h1"], r["h2"], lc.w["wg"][None], lc.w["wu"][None], lc.w["wd"][None],
                     lc.b, lc.c, rt["sel"], rt["g1"], rt["g2"])
    assert np.max(np.abs(got["out1"] - r["out1"])) <= 1e-12
    assert np.max(np.abs(got["out2"] - r["out2"])) <= 1e-12


def test_invariants():
    case, r1, r2 = tiny_case(5, TINY.replace(batch=4))
    rt = MO.route(r1, r2, TINY.k1, TINY.k2)
    base = run_ffn(case, rt)
    rng = np.random.default_rng(9)
    # the primary flow does not depend on the auxiliary flow's inputs, router logits or couplings
    rt_aux = MO.route(r1, rng.standard_normal(r2.shape), TINY.k1, TINY.k2)
    assert np.array_equal(rt_aux["sel"], rt["sel"]) and np.array_equal(rt_aux["g1"], rt["g1"])  # replay
    other = run_ffn(case, rt_aux, h2=rng.standard_normal(case.h2.shape), b=rng.standard_normal(TINY.mlp),
                    c=rng.standard_normal(TINY.hidden))
    assert np.array_equal(other["out1"], base["out1"])
    # relabelling the experts changes nothing
    perm = rng.permutation(TINY.experts)
    rp = MO.route(r1[:, perm], r2[:, perm], TINY.k1, TINY.k2)
    assert np.array_equal(perm[rp["sel"]], rt["sel"])
    pp = run_ffn(case, rp, wg=case.wg[perm], wu=case.wu[perm], wd=case.wd[perm])
    assert np.max(np.abs(pp["out1"] - base["out1"])) <= 1e-13 and np.max(np.abs(pp["out2"] - base["out2"])) <= 1e-13
    # equal flows, equal fan-outs, no coupling: the flows agree bit for bit
    rt_eq = MO.route(r1, r1, TINY.k1, TINY.k1)
    eq = run_ffn(case, rt_eq, h2=case.h1, res2=case.res1, b=None, c=None)
    assert np.array_equal(eq["out1"], eq["out2"])
    # c enters linearly through the primary's MoE output
    no_c = run_ffn(case, rt, c=None)
    assert np.max(np.abs(base["out2"] - no_c["out2"] - case.c * base["m1"])) <= 1e-14
    # equal auxiliary router logits: uniform auxiliary mixing weights
    flat = MO.route(r1, np.zeros_like(r2), TINY.k1, TINY.k2)
    assert np.allclose(flat["g2"], 1.0 / TINY.k2, rtol=0, atol=1e-16)
    assert np.allclose(rt["g1"].sum(-1), 1.0, rtol=0, atol=1e-15)
    # fan-outs: S1 is the prefix of S2, and a larger k2 extends S2 without reordering it
    wider = MO.route(r1, r2, TINY.k1, TINY.experts)
    assert np.array_equal(wider["sel"][:, :TINY.k2], rt["sel"])


@pytest.mark.parametrize("mistake", ["aux_own_router", "gates_over_all", "b_outside_s1", "c_from_aux"])
def test_planted_mistake_is_caught(mistake, monkeypatch):
    """A plausible error planted in the oracle fails at least one pin above."""
    real_route, real_ffn = MO.route, MO.moe_ffn

    def route(r1, r2, k1, k2):
        out = real_route(r1, r2, k1, k2)
        if mistake == "aux_own_router":
            out["sel"] = np.concatenate([out["sel"][:, :k1], np.argsort(-np.asarray(r2), axis=-1,
                                                                         kind="stable")[:, :k2 - k1]], axis=1)
        if mistake == "gates_over_all":
            out["g1"] = scipy.special.softmax(np.asarray(r1, dtype=np.float64), axis=-1)[
                np.arange(len(r1))[:, None], out["sel"][:, :k1]]
        return out

    def ffn(h1, h2, res1, res2, wg, wu, wd, b, c, sel, g1, g2):
        if mistake == "b_outside_s1" and b is not None:
            out = real_ffn(h1, h2, res1, res2, wg, wu, wd, b, c, sel, g1, g2)
            extra = np.zeros_like(out["m2"])
            for s in range(len(h1)):
                for slot in range(g1.shape[1], g2.shape[1]):
                    e = int(sel[s, slot])
                    z1 = MO.expert(np.asarray(h1[s:s + 1], dtype=np.float64), wg[e], wu[e])
                    extra[s] += g2[s, slot] * ((np.asarray(b) * z1) @ F.to_f64(wd[e], "bf16").T)[0]
            out["m2"] += extra
            out["out2"] = out["out2"] + extra
            return out
        out = real_ffn(h1, h2, res1, res2, wg, wu, wd, b, c, sel, g1, g2)
        if mistake == "c_from_aux" and c is not None:
            out["out2"] = out["out2"] + np.asarray(c) * (out["m2"] - out["m1"])
        return out

    monkeypatch.setattr(MO, "route", route)
    monkeypatch.setattr(MO, "moe_ffn", ffn)
    checks = [lambda: test_route_brute_force_with_ties(), lambda: test_route_matches_library_routines(),
              lambda: test_ffn_brute_force(3), test_single_expert_is_the_dense_layer_mlp, test_invariants]
    failed = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed >= 1
