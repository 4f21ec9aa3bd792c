"""Pins of oracle.stack: RMSNorm against torch and brute force, both rotary forms against complex
multiplication and RoPE's relative-position property, and the stack against the one-layer oracle."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as LY
from oracle import stack as ST

TINY = W.C5.replace(batch=2, hidden=16, num_q_heads=4, num_kv_heads=2, head_dim=8, mlp=24, ctx=20, block_size=16,
                    shuffle_blocks=True)


def test_rms_norm_matches_torch_and_brute_force():
    rng = np.random.default_rng(0)
    x, w = rng.standard_normal((3, 10)), rng.standard_normal(10)
    got = ST.rms_norm(x, w, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (10,), torch.from_numpy(w), eps=1e-5).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-14
    row = x[1].tolist()
    r = math.sqrt(math.fsum(v * v for v in row) / 10 + 1e-5)
    assert np.max(np.abs(got[1] - np.array([v / r * wi for v, wi in zip(row, w.tolist())]))) <= 1e-14


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_rope_is_complex_rotation(style):
    d, h, b = 8, 3, 2
    rng = np.random.default_rng(1)
    x = rng.standard_normal((b, h * d))
    cos, sin = ST.rope_tables(50, d)
    pos = np.array([0, 37])
    got = ST.rope(x, pos, cos, sin, d, style).reshape(b, h, d)
    xr = x.reshape(b, h, d)
    if style == "half":
        z = xr[..., :d // 2] + 1j * xr[..., d // 2:]
    else:
        z = xr[..., 0::2] + 1j * xr[..., 1::2]
    inv = 10000.0 ** (-np.arange(0, d, 2) / d)
    rot = z * np.exp(1j * pos[:, None, None] * inv[None, None, :])
    ref = np.concatenate([rot.real, rot.imag], -1) if style == "half" else \
        np.stack([rot.real, rot.imag], -1).reshape(b, h, d)
    assert np.max(np.abs(got - ref)) <= 1e-13
    assert np.array_equal(got[0], xr[0])  # position 0: no rotation


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_rope_scores_depend_on_relative_position(style):
    d = 16
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    cos, sin = ST.rope_tables(200, d)
    def score(m, n):
        return (ST.rope(q, np.array([m]), cos, sin, d, style) @ ST.rope(k, np.array([n]), cos, sin, d, style).T).item()
    assert abs(score(10, 3) - score(107, 100)) <= 1e-12
    assert abs(score(50, 50) - (q @ k.T).item()) <= 1e-12
    assert abs(score(10, 3) - score(3, 10)) > 1e-6  # not symmetric


def test_one_plain_layer_is_the_layer_oracle():
    cfg = W.StackConfig("one", TINY, layers=1, rope="none", rms=False)
    sc = W.make_stack_case(cfg, 61)
    lc = W.make_layer_case(TINY, 61)
    r = LY.dual_flow_layer(lc.x1, lc.x2, lc.w, lc.a, lc.b, lc.c, lc.k_cache, lc.v_cache, lc.block_table,
                           lc.ctx_lens, num_q_heads=TINY.num_q_heads, num_kv_heads=TINY.num_kv_heads,
                           head_dim=TINY.head_dim, scale=TINY.scale, block_size=lc.block_size)
    got = ST.stack_step(sc.x1, sc.x2, sc.layers, sc.k_caches, sc.v_caches, sc.block_table, sc.ctx_lens,
                        num_q_heads=TINY.num_q_heads, num_kv_heads=TINY.num_kv_heads, head_dim=TINY.head_dim,
                        scale=TINY.scale, block_size=sc.block_size)
    assert np.max(np.abs(got["out1"] - r["out1"])) <= 1e-12 and np.max(np.abs(got["out2"] - r["out2"])) <= 1e-12
    assert np.array_equal(got["caches"][0][0], r["k_cache"]) and np.array_equal(got["caches"][0][1], r["v_cache"])


def test_stack_invariants():
    cfg = W.StackConfig("three", TINY, layers=3, rope="half", rms=True)
    sc = W.make_stack_case(cfg, 62)
    kw = dict(num_q_heads=TINY.num_q_heads, num_kv_heads=TINY.num_kv_heads, head_dim=TINY.head_dim,
              scale=TINY.scale, block_size=sc.block_size, cos=sc.cos, sin=sc.sin, rms=True)
    got = ST.stack_step(sc.x1, sc.x2, sc.layers, sc.k_caches, sc.v_caches, sc.block_table, sc.ctx_lens,
                        rope_style="half", **kw)
    # the layers chain: two layers, then the third on their output
    two = ST.stack_step(sc.x1, sc.x2, sc.layers[:2], sc.k_caches, sc.v_caches, sc.block_table, sc.ctx_lens,
                        rope_style="half", **kw)
    third = ST.stack_step(two["out1"], two["out2"], sc.layers[2:], sc.k_caches[2:], sc.v_caches[2:],
                          sc.block_table, sc.ctx_lens, rope_style="half", **kw)
    assert np.array_equal(third["out1"], got["out1"]) and np.array_equal(third["out2"], got["out2"])
    # the primary flow never depends on the auxiliary flow
    alt = ST.stack_step(sc.x1, sc.x2 * -3.0, sc.layers, sc.k_caches, sc.v_caches, sc.block_table, sc.ctx_lens,
                        rope_style="half", **kw)
    assert np.array_equal(alt["out1"], got["out1"])
    for (k0, v0), (k1, v1) in zip(alt["caches"], got["caches"]):
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    # RMSNorm (without eps) ignores the scale of its input, and returns w where every entry is 1
    w = sc.layers[0]["n_attn"]
    assert np.max(np.abs(ST.rms_norm(2.5 * sc.x1, w, 0.0) - ST.rms_norm(sc.x1, w, 0.0))) <= 1e-14
    assert np.max(np.abs(ST.rms_norm(np.ones((1, TINY.hidden)), w, 0.0) - w)) <= 1e-15


def brute_stack(sc, style, rms, eps=1e-5):
    """Scalar loops: own matvec over struct-decoded bf16, complex-number rotations, math.fsum norms,
    explicit cache gathers, torch's bf16 rounding for the appended key/value."""
    import cmath
    import struct
    cfg = sc.cfg.layer
    D, Hq, Hkv = cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    bf = lambda bits: struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]
    def mv(w, x):
        return [math.fsum(bf(w[i, j]) * x[j] for j in range(len(x))) for i in range(w.shape[0])]
    def norm(x, w):
        if not rms:
            return list(x)
        r = math.sqrt(math.fsum(v * v for v in x) / len(x) + eps)
        return [v / r * float(wi) for v, wi in zip(x, w)]
    def rot(x, p):
        if style == "none":
            return list(x)
        y = list(x)
        for h in range(len(x) // D):
            for i in range(D // 2):
                ia, ib = (h * D + i, h * D + i + D // 2) if style == "half" else (h * D + 2 * i, h * D + 2 * i + 1)
                z = complex(x[ia], x[ib]) * cmath.exp(1j * p * 10000.0 ** (-2 * i / D))
                y[ia], y[ib] = z.real, z.imag
        return y
    def to_bf(vals):
        return torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).tolist()
    bs = sc.block_size
    x1s, x2s = [list(map(float, r)) for r in sc.x1], [list(map(float, r)) for r in sc.x2]
    for li, w in enumerate(sc.layers):
        n1, n2 = [], []
        for s in range(cfg.batch):
            L = int(sc.ctx_lens[s])
            a1, a2 = norm(x1s[s], w["n_attn"]), norm(x2s[s], w["n_attn"])
            q1, q2 = rot(mv(w["wq"], a1), L), rot(mv(w["wq"], a2), L)
            k1, v1 = to_bf(rot(mv(w["wk"], a1), L)), to_bf(mv(w["wv"], a1))
            o1, o2 = [], []
            for h in range(Hq):
                g = h // (Hq // Hkv)
                keys, vals = [], []
                for t in range(L):
                    blk, slot = int(sc.block_table[s, t // bs]), t % bs
                    keys.append([bf(sc.k_caches[li][blk, g, slot // 16, d // 8, slot % 16, d % 8]) for d in range(D)])
                    vals.append([bf(sc.v_caches[li][blk, g, slot // 16, d, slot % 16]) for d in range(D)])
                keys.append(k1[g * D:(g + 1) * D])
                vals.append(v1[g * D:(g + 1) * D])
                for f, q in ((1, q1), (2, q2)):
                    qq = [q[h * D + d] + (float(w["a"][h * D + d]) * q1[h * D + d] if f == 2 else 0.0) for d in range(D)]
                    sc_ = [cfg.scale * math.fsum(a * b for a, b in zip(qq, kk)) for kk in keys]
                    m = max(sc_)
                    e = [math.exp(v - m) for v in sc_]
                    tot = math.fsum(e)
                    out = [math.fsum(e[t] / tot * vals[t][d] for t in range(len(keys))) for d in range(D)]
                    (o1 if f == 1 else o2).extend(out)
            h1 = [a + b for a, b in zip(x1s[s], mv(w["wo"], o1))]
            h2 = [a + b for a, b in zip(x2s[s], mv(w["wo"], o2))]
            m1, m2 = norm(h1, w["n_mlp"]), norm(h2, w["n_mlp"])
            silu = lambda u: u / (1 + math.exp(-u))
            z1 = [silu(g) * u for g, u in zip(mv(w["wg"], m1), mv(w["wu"], m1))]
            z2 = [silu(g) * u + float(bb) * zz for g, u, bb, zz in zip(mv(w["wg"], m2), mv(w["wu"], m2), w["b"], z1)]
            d1 = mv(w["wd"], z1)
            n1.append([a + b for a, b in zip(h1, d1)])
            n2.append([a + b + float(cc) * dd for a, b, cc, dd in zip(h2, mv(w["wd"], z2), w["c"], d1)])
        x1s, x2s = n1, n2
    return np.array(x1s), np.array(x2s)


STYLES = [("half", True), ("interleaved", True), ("half", False), ("none", True)]


@pytest.mark.parametrize("style,rms", STYLES)
def test_stack_brute_force(style, rms):
    tiny = TINY.replace(ctx=5)
    cfg = W.StackConfig("b", tiny, layers=2, rope=style, rms=rms)
    sc = W.make_stack_case(cfg, 63)
    cos, sin = ST.rope_tables(sc.cos.shape[0], tiny.head_dim)
    got = ST.stack_step(sc.x1, sc.x2, sc.layers, sc.k_caches, sc.v_caches, sc.block_table, sc.ctx_lens,
                        num_q_heads=tiny.num_q_heads, num_kv_heads=tiny.num_kv_heads, head_dim=tiny.head_dim,
                        scale=tiny.scale, block_size=sc.block_size, rope_style=style, cos=cos, sin=sin, rms=rms)
    r1, r2 = brute_stack(sc, style, rms)
    assert np.max(np.abs(got["out1"] - r1)) <= 1e-10 and np.max(np.abs(got["out2"] - r2)) <= 1e-10


@pytest.mark.parametrize("mistake", ["no_rope_on_k", "rope_on_v", "norms_swapped", "q2_rotated_backwards"])
def test_planted_mistake_is_caught(mistake, monkeypatch):
    real_rope, real_linear, real_rms = ST.rope, ST.linear, ST.rms_norm
    state = {"n": 0}

    if mistake in ("no_rope_on_k", "q2_rotated_backwards"):
        def planted_rope(x, pos, cos, sin, head_dim, style):
            state["n"] += 1
            k = state["n"] % 3  # call order per layer: q1, q2, k1
            if mistake == "no_rope_on_k" and k == 0:
                return np.asarray(x, dtype=np.float64)
            if mistake == "q2_rotated_backwards" and k == 2:
                return real_rope(x, pos, cos, -np.asarray(sin), head_dim, style)
            return real_rope(x, pos, cos, sin, head_dim, style)
        monkeypatch.setattr(ST, "rope", planted_rope)
    elif mistake == "rope_on_v":
        calls = {"n": 0}
        def planted_linear(x, w_bits):
            out = real_linear(x, w_bits)
            calls["n"] += 1
            if calls["n"] % 12 == 4:  # per layer: wq, wq, wk, wv, wo, wo, wg, wu, wg, wu, wd, wd
                out = real_rope(out, np.full(out.shape[0], 3), *ST.rope_tables(64, TINY.head_dim), TINY.head_dim, "half")
            return out
        monkeypatch.setattr(ST, "linear", planted_linear)
    else:
        def planted_rms(x, w, eps):
            return real_rms(x, np.asarray(w)[::-1], eps)
        monkeypatch.setattr(ST, "rms_norm", planted_rms)
    failed = 0
    for style, rms in STYLES[:2]:
        try:
            test_stack_brute_force(style, rms)
        except AssertionError:
            failed += 1
    assert failed >= 1
