"""GPU parity of dfa_pack_weight, dfa_dual_gemv and dfa_decode_layer with the oracle.

The GEMV epilogues are checked against the oracle's layer steps (linear,
silu, couple, bf16 append) on ragged batches and several split-K plans; the
whole layer against oracle.layer.dual_flow_layer on a reduced shape and on the
full workload (batch 32, hidden 4096, 32/8 heads of 128, MLP 14336, 4096 cached
positions). Invariants: the primary flow's outputs and the cache do not depend
on the auxiliary flow's inputs; without coupling and with x2 = x1 the flows
agree; the cache changes only at the appended position, within one bf16 ulp of
the oracle's rounding of k1 and v1.
"""
import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import TOL, assert_close, say
from oracle import formats as F
from oracle import layer as LY
from workloads.device import to_device

pytestmark = pytest.mark.gpu


def pack(w_bits):
    n, k = w_bits.shape
    w = to_device(w_bits)
    wt = torch.empty_like(w)
    dfa.dfa_pack_weight(w, wt, n, k)
    return wt


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in bf16 ulps between two arrays of finite bf16 bit patterns."""
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def test_pack_weight_layout():
    rng = np.random.default_rng(0)
    w = rng.integers(0, 1 << 16, size=(48, 40), dtype=np.uint16)
    say("case pack weight")
    got = pack(w).cpu().numpy().view(np.uint16).reshape(-1)
    ref = w.reshape(3, 16, 5, 8).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(got, ref)


def gemv(epi, w_bits, x1, x2=None, w2_bits=None, couple=None, res1=None, res2=None, x_exact=0, k_split=0,
         kv=None, y_kv=False, rows=0):
    n, k = w_bits.shape
    flows = 1 if x2 is None else 2
    batch = x1.shape[0]
    d = dfa.GemvDesc(batch=batch, n=n, k=k, num_flows=flows, epilogue=epi, x_exact_bf16=x_exact, k_split=k_split,
                     rows_per_wg=rows)
    ws = torch.empty(max(dfa.dfa_dual_gemv_workspace_size(d) // 4, 4), dtype=torch.float32, device="cuda")
    t = lambda a: None if a is None else to_device(np.ascontiguousarray(a, dtype=np.float32))
    y1 = torch.full((batch, n), float("nan"), device="cuda") if (epi != dfa.DFA_EPI_KV_APPEND or y_kv) else None
    y2 = torch.full((batch, n), float("nan"), device="cuda") if (flows == 2 or y_kv) else None
    dfa.dfa_dual_gemv(d, pack(w_bits), None if w2_bits is None else pack(w2_bits), t(x1), t(x2), t(couple), t(res1),
                      t(res2), y1, y2, kv, ws)
    torch.cuda.synchronize()
    return (None if y1 is None else y1.cpu().numpy()), (None if y2 is None else y2.cpu().numpy())


def rand_w(rng, n, k, std=0.02):
    return W.f32_to_bf16_bits(rng.standard_normal((n, k)).astype(np.float32) * np.float32(std))


@pytest.mark.parametrize("batch,k_split,rows", [(1, 0, 0), (17, 0, 0), (32, 1, 0), (32, 2, 0), (5, 3, 0),
                                               (32, 1, 128), (17, 2, 128), (1, 3, 128),
                                               # beyond 32 sequences: slices of 32 (the last one ragged)
                                               (40, 0, 0), (70, 2, 0), (64, 1, 128)])
def test_gemv_epilogues(batch, k_split, rows):
    rng = np.random.default_rng(batch * 10 + k_split)
    n, k = 256, 384
    x1, x2 = rng.standard_normal((2, batch, k)).astype(np.float32)
    r1, r2 = rng.standard_normal((2, batch, n)).astype(np.float32)
    cpl = rng.standard_normal(n).astype(np.float32) * np.float32(0.1)
    w, w2 = rand_w(rng, n, k), rand_w(rng, n, k)
    x1d, x2d = x1.astype(np.float64), x2.astype(np.float64)
    say(f"case gemv batch={batch} k_split={k_split} rows={rows}")
    y1, y2 = gemv(dfa.DFA_EPI_NONE, w, x1, x2, k_split=k_split, rows=rows)
    assert_close(y1, LY.linear(x1d, w), what="none y1")
    assert_close(y2, LY.linear(x2d, w), what="none y2")
    y1, y2 = gemv(dfa.DFA_EPI_RESIDUAL, w, x1, x2, res1=r1, res2=r2, k_split=k_split, rows=rows)
    assert_close(y1, r1 + LY.linear(x1d, w), what="residual y1")
    assert_close(y2, r2 + LY.linear(x2d, w), what="residual y2")
    y1, y2 = gemv(dfa.DFA_EPI_SWIGLU, w, x1, x2, w2_bits=w2, couple=cpl, k_split=k_split, rows=rows)
    z1 = LY.silu(LY.linear(x1d, w)) * LY.linear(x1d, w2)
    z2 = LY.couple(LY.silu(LY.linear(x2d, w)) * LY.linear(x2d, w2), cpl.astype(np.float64), z1)
    assert_close(y1, z1, what="swiglu z1")
    assert_close(y2, z2, what="swiglu z2'")
    y1, y2 = gemv(dfa.DFA_EPI_RESIDUAL_COUPLED, w, x1, x2, couple=cpl, res1=r1, res2=r2, k_split=k_split,
                  rows=rows)
    m1 = LY.linear(x1d, w)
    assert_close(y1, r1 + m1, what="coupled y1")
    assert_close(y2, r2 + LY.couple(LY.linear(x2d, w), cpl.astype(np.float64), m1), what="coupled y2")


@pytest.mark.parametrize("k_split", [0, 32])
def test_gemv_many_k_ranges(k_split):
    """64 x 4096, the shape of a MoE router: the library's choice (16 k-ranges, all of a reduction
    thread's loads at once) and 32 k-ranges (the reduction's general path)."""
    rng = np.random.default_rng(31 + k_split)
    n, k = 64, 4096
    x1, x2 = rng.standard_normal((2, 32, k)).astype(np.float32)
    r1, r2 = rng.standard_normal((2, 32, n)).astype(np.float32)
    cpl = rng.standard_normal(n).astype(np.float32) * np.float32(0.1)
    w = rand_w(rng, n, k)
    x1d, x2d = x1.astype(np.float64), x2.astype(np.float64)
    say(f"case gemv 64 x 4096 k_split={k_split}")
    y1, y2 = gemv(dfa.DFA_EPI_NONE, w, x1, x2, k_split=k_split)
    assert_close(y1, LY.linear(x1d, w), what="router y1")
    assert_close(y2, LY.linear(x2d, w), what="router y2")
    y1, y2 = gemv(dfa.DFA_EPI_RESIDUAL_COUPLED, w, x1, x2, couple=cpl, res1=r1, res2=r2, k_split=k_split)
    m1 = LY.linear(x1d, w)
    assert_close(y1, r1 + m1, what="router coupled y1")
    assert_close(y2, r2 + LY.couple(LY.linear(x2d, w), cpl.astype(np.float64), m1), what="router coupled y2")


@pytest.mark.parametrize("k_split", [1, 3])
def test_gemv_rows_multiple_of_64(k_split):
    rng = np.random.default_rng(11 + k_split)
    x1, x2 = rng.standard_normal((2, 7, 384)).astype(np.float32)
    w = rand_w(rng, 192, 384)
    say(f"case gemv n=192 k_split={k_split}")
    y1, y2 = gemv(dfa.DFA_EPI_NONE, w, x1, x2, k_split=k_split)
    assert_close(y1, LY.linear(x1.astype(np.float64), w), what="n=192 y1")
    assert_close(y2, LY.linear(x2.astype(np.float64), w), what="n=192 y2")


@pytest.mark.parametrize("batch", [40, 64, 100])
def test_gemv_one_flow_wide_batch(batch):
    rng = np.random.default_rng(batch)
    x1 = rng.standard_normal((batch, 256)).astype(np.float32)
    w = rand_w(rng, 128, 256)
    say(f"case gemv one flow batch={batch}")
    y1, _ = gemv(dfa.DFA_EPI_NONE, w, x1)
    assert_close(y1, LY.linear(x1.astype(np.float64), w), what="one-flow y1")


@pytest.mark.parametrize("k_split", [1, 2])
def test_gemv_zero_weights_return_the_residual(k_split):
    rng = np.random.default_rng(21 + k_split)
    x1, x2 = rng.standard_normal((2, 9, 256)).astype(np.float32)
    r1, r2 = rng.standard_normal((2, 9, 128)).astype(np.float32)
    cpl = rng.standard_normal(128).astype(np.float32)
    w = np.zeros((128, 256), dtype=np.uint16)  # +0.0 in bf16
    say(f"case gemv zero weights k_split={k_split}")
    y1, y2 = gemv(dfa.DFA_EPI_RESIDUAL, w, x1, x2, res1=r1, res2=r2, k_split=k_split)
    assert np.array_equal(y1, r1) and np.array_equal(y2, r2)
    y1, y2 = gemv(dfa.DFA_EPI_RESIDUAL_COUPLED, w, x1, x2, couple=cpl, res1=r1, res2=r2, k_split=k_split)
    assert np.array_equal(y1, r1) and np.array_equal(y2, r2)


def test_exact_bf16_activations_skip_low_halves():
    rng = np.random.default_rng(7)
    x1, x2 = (W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((2, 9, 512)).astype(np.float32))))
    w = rand_w(rng, 384, 512)
    say("case gemv exact bf16")
    a1, a2 = gemv(dfa.DFA_EPI_NONE, w, x1, x2, x_exact=0)
    b1, b2 = gemv(dfa.DFA_EPI_NONE, w, x1, x2, x_exact=1)
    assert np.array_equal(a1, b1) and np.array_equal(a2, b2)
    assert_close(b1, LY.linear(x1.astype(np.float64), w), what="exact y1")


@pytest.mark.parametrize("k_split,batch", [(1, 5), (2, 5), (2, 70)])
def test_gemv_kv_append(k_split, batch):
    """The primary-only append, in the GEMV kernel (one k-range) and after the split reduction; 70
    sequences run in slices of 64."""
    cfg = SMALL_LAYER.replace(num_kv_heads=2, hidden=384, batch=batch)
    case = W.make_layer_case(cfg, 40 + k_split + batch)
    kd = cfg.num_kv_heads * cfg.head_dim
    k_cache, v_cache = to_device(case.k_cache), to_device(case.v_cache)
    table, ctx = to_device(case.block_table), to_device(case.ctx_lens)  # kept alive: kv holds raw addresses
    kv = dfa.kv_target(k_cache, v_cache, table, ctx, cfg.num_kv_heads, cfg.head_dim, case.block_size,
                       case.max_blocks_per_seq, case.k_cache.shape[0])
    say(f"case gemv kv append k_split={k_split} batch={batch}")
    y1, y2 = gemv(dfa.DFA_EPI_KV_APPEND, case.w["wk"], case.x1, w2_bits=case.w["wv"], x_exact=1, k_split=k_split,
                  kv=kv, y_kv=True)
    k_lin, v_lin = LY.linear(case.x1, case.w["wk"]), LY.linear(case.x1, case.w["wv"])
    assert_close(y1, k_lin, what="appended k as float32")
    assert_close(y2, v_lin, what="appended v as float32")
    shape = (cfg.batch, cfg.num_kv_heads, cfg.head_dim)
    ref_k, ref_v = LY.append_kv(case.k_cache, case.v_cache, case.block_table, case.ctx_lens,
                                F.f64_to_bf16_bits(k_lin).reshape(shape), F.f64_to_bf16_bits(v_lin).reshape(shape),
                                case.block_size)
    n_app = cfg.batch * kd
    for name, g, r, orig in (("k", k_cache, ref_k, case.k_cache), ("v", v_cache, ref_v, case.v_cache)):
        g = g.cpu().numpy().view(np.uint16)
        diff = g != r
        assert diff.sum() <= n_app, name
        if diff.any():
            assert bf16_ulp_diff(g[diff], r[diff]).max() <= 1, name
        assert (g != orig).sum() <= n_app, name


def test_gemv_rejects_bad_shapes():
    d = dfa.GemvDesc(batch=65536, n=128, k=128, num_flows=2, epilogue=0, x_exact_bf16=0, k_split=0)
    assert dfa.dfa_dual_gemv_workspace_size(d) == 0
    d = dfa.GemvDesc(batch=4, n=96, k=128, num_flows=2, epilogue=0, x_exact_bf16=0, k_split=2)
    assert dfa.dfa_dual_gemv_workspace_size(d) == 0
    d = dfa.GemvDesc(batch=4, n=192, k=128, num_flows=2, epilogue=0, x_exact_bf16=0, k_split=1)
    assert dfa.dfa_dual_gemv_workspace_size(d) == 0  # valid; one k-range needs no workspace
    d = dfa.GemvDesc(batch=4, n=192, k=256, num_flows=2, epilogue=0, x_exact_bf16=0, k_split=2)
    assert dfa.dfa_dual_gemv_workspace_size(d) == 2 * 32 * 192 * 4  # 2 splits x 2 flows x 16 padded rows
    for rows, n in ((96, 256), (128, 192)):  # not 0/64/128; 128 rows need n % 128 == 0
        d = dfa.GemvDesc(batch=4, n=n, k=256, num_flows=2, epilogue=0, x_exact_bf16=0, k_split=2, rows_per_wg=rows)
        assert dfa.dfa_dual_gemv_workspace_size(d) == 0


# ---------------------------------------------------------------- full layer
def layer_inputs(case):
    cfg = case.cfg
    packed = {name: pack(case.w[name]) for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}
    dev = {"x1": to_device(case.x1), "x2": to_device(case.x2), "a": to_device(case.a), "b": to_device(case.b),
           "c": to_device(case.c), "k": to_device(case.k_cache), "v": to_device(case.v_cache),
           "table": to_device(case.block_table), "ctx": to_device(case.ctx_lens)}
    desc = dfa.LayerDesc(batch=cfg.batch, hidden=cfg.hidden, num_q_heads=cfg.num_q_heads,
                         num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, mlp=cfg.mlp,
                         block_size=case.block_size, max_blocks_per_seq=case.max_blocks_per_seq,
                         num_blocks=case.k_cache.shape[0], max_ctx_len=int(case.ctx_lens.max()) + 1,
                         scale=cfg.scale, x_exact_bf16=1)
    return packed, dev, desc


def run_layer(case, packed, dev, desc, **override):
    d = dict(dev)
    d.update(override)
    wts = dfa.layer_weights(packed["wq"], packed["wk"], packed["wv"], packed["wo"], packed["wg"], packed["wu"],
                            packed["wd"], d["a"], d["b"], d["c"])
    ws = torch.empty(dfa.dfa_decode_layer_workspace_size(desc) // 4 + 64, dtype=torch.float32, device="cuda")
    out1 = torch.full(tuple(case.x1.shape), float("nan"), device="cuda")
    out2 = torch.full_like(out1, float("nan"))
    k, v = d["k"].clone(), d["v"].clone()
    dfa.dfa_decode_layer(desc, wts, d["x1"], d["x2"], k, v, d["table"], d["ctx"], out1, out2, ws)
    torch.cuda.synchronize()
    return out1.cpu().numpy(), out2.cpu().numpy(), k.cpu().numpy().view(np.uint16), v.cpu().numpy().view(np.uint16)


def oracle_layer(case):
    cfg = case.cfg
    return LY.dual_flow_layer(case.x1, case.x2, case.w, case.a, case.b, case.c, case.k_cache, case.v_cache,
                              case.block_table, case.ctx_lens, num_q_heads=cfg.num_q_heads,
                              num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, scale=cfg.scale,
                              block_size=case.block_size)


def check_layer(case, got, ref, label):
    out1, out2, k, v = got
    assert_close(out1, ref["out1"], what=f"{label} out1")
    assert_close(out2, ref["out2"], what=f"{label} out2")
    # the cache differs from the oracle's only at appended slots, and there by at most 1 bf16 ulp
    n_app = k1v1_count(case)
    for name, g, r in (("k", k, ref["k_cache"]), ("v", v, ref["v_cache"])):
        diff = g != r
        say(f"  {label}: appended {name} bits equal to the oracle's for {100 * (1 - diff.sum() / n_app):.3f}%")
        assert diff.sum() <= n_app
        if diff.any():
            assert bf16_ulp_diff(g[diff], r[diff]).max() <= 1
    # and nothing but the appended slots changed
    assert (k != case.k_cache).sum() <= n_app and (v != case.v_cache).sum() <= n_app


def k1v1_count(case):
    return case.cfg.batch * case.cfg.num_kv_heads * case.cfg.head_dim


SMALL_LAYER = W.C5.replace(batch=5, hidden=256, num_q_heads=4, num_kv_heads=1, head_dim=128, mlp=384, ctx=300,
                           block_size=16, shuffle_blocks=True)


def test_layer_small_paged():
    case = W.make_layer_case(SMALL_LAYER, 31)
    packed, dev, desc = layer_inputs(case)
    say("case layer small paged")
    check_layer(case, run_layer(case, packed, dev, desc), oracle_layer(case), "small layer")


def test_layer_batch_beyond_32():
    """40 sequences: the GEMVs (and the fused QKV append) run in slices of 32, attention over all 40."""
    case = W.make_layer_case(SMALL_LAYER.replace(batch=40), 32)
    packed, dev, desc = layer_inputs(case)
    say("case layer batch 40")
    check_layer(case, run_layer(case, packed, dev, desc), oracle_layer(case), "batch-40 layer")


def test_layer_sixteen_heads_per_kv_head():
    """16 query heads per kv head: attention runs 32 query rows (both flows) per kv head."""
    cfg = SMALL_LAYER.replace(num_q_heads=32, num_kv_heads=2, head_dim=64, hidden=512, batch=3)
    case = W.make_layer_case(cfg, 33)
    packed, dev, desc = layer_inputs(case)
    say("case layer 16 heads per kv head")
    check_layer(case, run_layer(case, packed, dev, desc), oracle_layer(case), "g16 layer")


@pytest.mark.slow
def test_layer_full_size():
    say("case layer full size (c5): generating inputs")
    case = W.make_layer_case(W.C5, W.SEEDS["c5"])
    packed, dev, desc = layer_inputs(case)
    say("case layer full size: running the GPU")
    got = run_layer(case, packed, dev, desc)
    say("case layer full size: running the oracle")
    check_layer(case, got, oracle_layer(case), "c5 layer")


def test_layer_primary_independent_of_aux_flow():
    case = W.make_layer_case(SMALL_LAYER, 32)
    packed, dev, desc = layer_inputs(case)
    say("case layer primary independence")
    ref = run_layer(case, packed, dev, desc)
    g = torch.Generator(device="cuda").manual_seed(3)
    other = {"x2": torch.randn(dev["x2"].shape, device="cuda", generator=g),
             "a": torch.randn(dev["a"].shape, device="cuda", generator=g),
             "b": torch.randn(dev["b"].shape, device="cuda", generator=g),
             "c": torch.randn(dev["c"].shape, device="cuda", generator=g)}
    got = run_layer(case, packed, dev, desc, **other)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[2], got[2]) and np.array_equal(ref[3], got[3])
    assert not np.array_equal(ref[1], got[1])


def test_layer_aux_equals_primary_without_coupling():
    case = W.make_layer_case(SMALL_LAYER, 33)
    packed, dev, desc = layer_inputs(case)
    say("case layer aux == primary")
    z = torch.zeros_like
    out1, out2, _, _ = run_layer(case, packed, dev, desc, x2=dev["x1"].clone(), a=z(dev["a"]), b=z(dev["b"]),
                                 c=z(dev["c"]))
    assert np.array_equal(out1, out2)
