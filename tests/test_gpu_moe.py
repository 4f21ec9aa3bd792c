"""GPU parity of dfa_moe_route and dfa_moe_ffn (router replay, grouped expert GEMVs) with oracle.moe.

Routing: the selection is compared exactly (integer work), the mixing weights to 1e-6. The FFN
outputs: the row-normalised max relative error of the other GPU tests (2e-3) against the float64
oracle run on the same routing. Invariants: the primary flow is bit for bit independent of the
auxiliary flow's inputs; with equal flows, equal fan-outs and no coupling the flows agree bit for
bit. Edge cases: one sequence, ragged batches (17: two activation blocks per flow; 70: slices of
32), one expert, every expert selected, an expert chosen by every sequence, experts chosen by none,
inputs that are not exact bf16 values, NULL couplings and residuals. The full workload (batch 32, hidden 4096, 64
experts of width 1024, fan-outs 4 and 8) is checked on every sequence.
"""
import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import TOL, assert_close, say
from oracle import formats as F
from oracle import moe as MO
from workloads.device import to_device

pytestmark = pytest.mark.gpu


def pack_experts(w_bits):
    """[E, n, k] bf16 bits -> the experts' tiled matrices back to back on the GPU."""
    ne, n, k = w_bits.shape
    src = to_device(np.ascontiguousarray(w_bits))
    dst = torch.empty_like(src)
    for e in range(ne):
        dfa.dfa_pack_weight(src[e], dst[e], n, k)
    return dst


def router_logits(case):
    wr = F.to_f64(case.wr, "bf16")
    return (case.h1 @ wr.T).astype(np.float32), (case.h2 @ wr.T).astype(np.float32)


def desc_of(cfg, x_exact=1):
    return dfa.MoeDesc(batch=cfg.batch, hidden=cfg.hidden, mlp=cfg.mlp, num_experts=cfg.experts, k1=cfg.k1,
                       k2=cfg.k2, x_exact_bf16=x_exact)


def gpu_route(d, r1, r2):
    routing = torch.zeros(dfa.dfa_moe_routing_size(d) // 4, dtype=torch.int32, device="cuda")
    dfa.dfa_moe_route(d, to_device(np.ascontiguousarray(r1)), to_device(np.ascontiguousarray(r2)), routing)
    torch.cuda.synchronize()
    raw = routing.cpu().numpy()
    b, k1, k2 = d.batch, d.k1, d.k2
    up4 = lambda x: (x + 3) // 4 * 4
    sel = raw[:b * k2].reshape(b, k2)
    o1 = up4(b * k2)
    g1 = raw[o1:o1 + b * k1].view(np.float32).reshape(b, k1)
    o2 = o1 + up4(b * k1)
    g2 = raw[o2:o2 + b * k2].view(np.float32).reshape(b, k2)
    return routing, sel, g1, g2


class Dev:
    """A case's weights and couplings on the GPU."""

    def __init__(self, case):
        self.wg, self.wu, self.wd = pack_experts(case.wg), pack_experts(case.wu), pack_experts(case.wd)
        self.b, self.c = to_device(case.b), to_device(case.c)


def gpu_ffn(d, dev, routing, h1, h2, res1, res2, b=True, c=True):
    ws = torch.full((dfa.dfa_moe_workspace_size(d) // 4,), float("nan"), device="cuda")
    t = lambda a: None if a is None else to_device(np.ascontiguousarray(a, dtype=np.float32))
    out1 = torch.full((d.batch, d.hidden), float("nan"), device="cuda")
    out2 = torch.full_like(out1, float("nan"))
    dfa.dfa_moe_ffn(d, dev.wg, dev.wu, dev.wd, dev.b if b else None, dev.c if c else None, t(h1), t(h2), t(res1),
                    t(res2), routing, out1, out2, ws)
    torch.cuda.synchronize()
    return out1.cpu().numpy(), out2.cpu().numpy()


def check_route(d, r1, r2, what):
    routing, sel, g1, g2 = gpu_route(d, r1, r2)
    ref = MO.route(r1, r2, d.k1, d.k2)
    assert np.array_equal(sel, ref["sel"]), f"{what}: selection"
    e1, e2 = np.max(np.abs(g1 - ref["g1"])), np.max(np.abs(g2 - ref["g2"]))
    say(f"  {what}: selection exact, mixing weights max err {max(e1, e2):.2e}")
    assert e1 <= 1e-6 and e2 <= 1e-6
    return routing, ref


@pytest.mark.parametrize("batch,experts,k1,k2,ties", [(1, 1, 1, 1, False), (5, 9, 2, 4, False), (32, 64, 4, 8, False),
                                                      (7, 16, 3, 3, True), (3, 1024, 8, 32, False),
                                                      (32, 5, 5, 5, True)])
def test_route_matches_oracle(batch, experts, k1, k2, ties):
    rng = np.random.default_rng(experts + k2)
    if ties:
        r1 = rng.integers(-2, 2, size=(batch, experts)).astype(np.float32)
    else:
        r1 = rng.standard_normal((batch, experts), dtype=np.float32)
    r2 = rng.standard_normal((batch, experts), dtype=np.float32)
    d = dfa.MoeDesc(batch=batch, hidden=128, mlp=128, num_experts=experts, k1=k1, k2=k2, x_exact_bf16=1)
    say(f"case route batch {batch} experts {experts} k1 {k1} k2 {k2} ties {ties}")
    check_route(d, r1, r2, "route")


SMALL = {
    "b5": W.MoeConfig("b5", batch=5, hidden=256, mlp=128, experts=6, k1=2, k2=4, w_std=0.05),
    "b17": W.MoeConfig("b17", batch=17, hidden=384, mlp=256, experts=9, k1=1, k2=3, w_std=0.05),
    "b1": W.MoeConfig("b1", batch=1, hidden=128, mlp=384, experts=3, k1=2, k2=3, w_std=0.05),
    "equal_fanout": W.MoeConfig("eq", batch=12, hidden=256, mlp=128, experts=8, k1=3, k2=3, w_std=0.05),
    "all_experts": W.MoeConfig("all", batch=32, hidden=128, mlp=128, experts=4, k1=2, k2=4, w_std=0.05),
    "one_expert": W.MoeConfig("one", batch=9, hidden=256, mlp=256, experts=1, k1=1, k2=1, w_std=0.05),
    "max_fanout": W.MoeConfig("wide", batch=3, hidden=128, mlp=128, experts=40, k1=1, k2=32, w_std=0.05),
    "max_experts": W.MoeConfig("e1024", batch=6, hidden=128, mlp=128, experts=1024, k1=2, k2=8, w_std=0.05),
    # beyond 32 sequences: the expert GEMVs and the combination run in slices of 32 (the last one ragged)
    "b70": W.MoeConfig("b70", batch=70, hidden=256, mlp=128, experts=8, k1=2, k2=4, w_std=0.05),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_moe_ffn_matches_oracle(name):
    cfg = SMALL[name]
    case = W.make_moe_case(cfg, 41)
    r1, r2 = router_logits(case)
    d = desc_of(cfg)
    say(f"case moe {name}: batch {cfg.batch} hidden {cfg.hidden} mlp {cfg.mlp} experts {cfg.experts} "
        f"k1 {cfg.k1} k2 {cfg.k2}")
    routing, rt = check_route(d, r1, r2, name)
    dev = Dev(case)
    o1, o2 = gpu_ffn(d, dev, routing, case.h1, case.h2, case.res1, case.res2)
    ref = MO.moe_ffn(case.h1, case.h2, case.res1, case.res2, case.wg, case.wu, case.wd, case.b, case.c,
                     rt["sel"], rt["g1"], rt["g2"])
    assert_close(o1, ref["out1"], TOL, f"{name} out1")
    assert_close(o2, ref["out2"], TOL, f"{name} out2")
    assert_close(o1 - case.res1, ref["m1"], TOL, f"{name} m1")


def test_inputs_not_bf16_and_null_terms():
    cfg = SMALL["b17"]
    case = W.make_moe_case(cfg, 43)
    rng = np.random.default_rng(3)
    h1 = rng.standard_normal(case.h1.shape).astype(np.float32)  # not exact bf16: hi/lo split
    h2 = rng.standard_normal(case.h2.shape).astype(np.float32)
    r1, r2 = router_logits(case)
    d = desc_of(cfg, x_exact=0)
    say("case moe: float32 inputs, no couplings, no residuals")
    routing, rt = check_route(d, r1, r2, "f32 inputs")
    o1, o2 = gpu_ffn(d, Dev(case), routing, h1, h2, None, None, b=False, c=False)
    ref = MO.moe_ffn(h1, h2, np.zeros_like(h1), np.zeros_like(h2), case.wg, case.wu, case.wd, None, None,
                     rt["sel"], rt["g1"], rt["g2"])
    assert_close(o1, ref["out1"], TOL, "out1")
    assert_close(o2, ref["out2"], TOL, "out2")


def test_one_expert_for_everyone_and_idle_experts():
    """Expert 3 heads every sequence's ranking (its list holds the whole batch of 32); most other
    experts are chosen by nobody (their workgroups exit at once)."""
    cfg = W.MoeConfig("crowd", batch=32, hidden=256, mlp=128, experts=12, k1=1, k2=2, w_std=0.05)
    case = W.make_moe_case(cfg, 45)
    r1, r2 = router_logits(case)
    r1[:, 3] = 50.0
    r1[:, 7] = 40.0
    d = desc_of(cfg)
    say("case moe: one expert for every sequence")
    routing, rt = check_route(d, r1, r2, "crowd")
    assert np.all(rt["sel"][:, 0] == 3) and np.all(rt["sel"][:, 1] == 7)
    o1, o2 = gpu_ffn(d, Dev(case), routing, case.h1, case.h2, case.res1, case.res2)
    ref = MO.moe_ffn(case.h1, case.h2, case.res1, case.res2, case.wg, case.wu, case.wd, case.b, case.c,
                     rt["sel"], rt["g1"], rt["g2"])
    assert_close(o1, ref["out1"], TOL, "out1")
    assert_close(o2, ref["out2"], TOL, "out2")


def test_invariants():
    cfg = SMALL["b5"]
    case = W.make_moe_case(cfg, 47)
    r1, r2 = router_logits(case)
    d = desc_of(cfg)
    dev = Dev(case)
    say("case moe invariants")
    routing, _ = gpu_route(d, r1, r2)[:2]
    o1, o2 = gpu_ffn(d, dev, routing, case.h1, case.h2, case.res1, case.res2)
    # the primary flow ignores the auxiliary flow's inputs, router logits and couplings
    rng = np.random.default_rng(8)
    routing_b = gpu_route(d, r1, rng.standard_normal(r2.shape).astype(np.float32) * 4)[0]
    dev_b = Dev(case)
    dev_b.b = to_device(rng.standard_normal(cfg.mlp).astype(np.float32))
    dev_b.c = to_device(rng.standard_normal(cfg.hidden).astype(np.float32))
    h2b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal(case.h2.shape).astype(np.float32) * 3))
    p1, p2 = gpu_ffn(d, dev_b, routing_b, case.h1, h2b, case.res1, case.res1 * 2)
    assert np.array_equal(p1, o1)
    assert not np.array_equal(p2, o2)
    # equal flows, equal fan-outs, no couplings: bit for bit equal
    d_eq = dfa.MoeDesc(batch=cfg.batch, hidden=cfg.hidden, mlp=cfg.mlp, num_experts=cfg.experts, k1=cfg.k2,
                       k2=cfg.k2, x_exact_bf16=1)
    routing_eq = gpu_route(d_eq, r1, r1)[0]
    e1, e2 = gpu_ffn(d_eq, dev, routing_eq, case.h1, case.h1, case.res1, case.res1, b=False, c=False)
    assert np.array_equal(e1, e2)
    # repeated calls agree bit for bit
    q1, q2 = gpu_ffn(d, dev, routing, case.h1, case.h2, case.res1, case.res2)
    assert np.array_equal(q1, o1) and np.array_equal(q2, o2)


def test_full_workload_all_sequences():
    """The full workload (batch 32, hidden 4096, 64 experts of width 1024, fan-outs 4 and 8): every
    sequence of both flows against the oracle (about 15 s of oracle time)."""
    cfg = W.MOE
    say("case moe full size: generating inputs")
    case = W.make_moe_case(cfg, W.SEEDS["moe"])
    r1, r2 = router_logits(case)
    d = desc_of(cfg)
    routing, rt = check_route(d, r1, r2, "moe full")
    dev = Dev(case)
    say("case moe full size: running the GPU")
    o1, o2 = gpu_ffn(d, dev, routing, case.h1, case.h2, case.res1, case.res2)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(o2))
    say("case moe full size: oracle over all 32 sequences")
    ref = MO.moe_ffn(case.h1, case.h2, case.res1, case.res2, case.wg, case.wu, case.wd, case.b, case.c, rt["sel"],
                     rt["g1"], rt["g2"])
    assert_close(o1, ref["out1"], TOL, "moe out1 (all sequences)")
    assert_close(o2, ref["out2"], TOL, "moe out2 (all sequences)")
    assert_close(o1 - case.res1, ref["m1"], TOL, "moe m1 (all sequences)")


def test_route_with_nan_logits_selects_distinct_experts():
    """NaN router logits (outside the header's contract) still give a valid routing: the ranking
    reads NaN as -inf with ties to the smaller index, so every selection is k2 distinct experts in
    range, the finite experts come first in descending order, and rows without NaN match the
    oracle (regression: NaN once gave several experts one rank and repeated an expert)."""
    rng = np.random.default_rng(404)
    batch, experts, k1, k2 = 6, 12, 3, 8
    r1 = rng.standard_normal((batch, experts), dtype=np.float32)
    r2 = rng.standard_normal((batch, experts), dtype=np.float32)
    r1[1, [0, 5]] = np.nan
    r1[2, :] = np.nan
    r1[4, 3:] = np.nan  # only 3 finite experts, fewer than k2
    d = dfa.MoeDesc(batch=batch, hidden=128, mlp=128, num_experts=experts, k1=k1, k2=k2, x_exact_bf16=1)
    say("case route with NaN router logits")
    _, sel, _, _ = gpu_route(d, r1, r2)
    for b in range(batch):
        row = sel[b]
        assert len(set(row.tolist())) == k2 and row.min() >= 0 and row.max() < experts, (b, row)
        key = np.where(np.isnan(r1[b]), -np.inf, r1[b]).astype(np.float64)
        order = sorted(range(experts), key=lambda e: (-key[e], e))
        assert row.tolist() == order[:k2], (b, row, order[:k2])
    clean = np.array([0, 3, 5])
    ref = MO.route(r1[clean], r2[clean], k1, k2)
    assert np.array_equal(sel[clean], ref["sel"])
