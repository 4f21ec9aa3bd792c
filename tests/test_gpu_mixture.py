"""GPU parity of dfa_mixture_sample (and of the dual output head feeding it) with oracle.mixture.

Per sequence the library returns alpha, optionally p_mix, the greedy token and
the inverse-CDF token for the caller's uniform u. Bars:

* alpha: absolute error <= 5e-5 (fixed-order float32 sums: one reduction over
  at most 32768 tokens, or at most 256 chunk records of 4096 tokens each, the
  two paths split at 32768 tokens: relative error ~1e-6);
* p_mix: the row-normalised max relative error of the other GPU tests (2e-3);
* greedy: the oracle's argmax, unless the oracle's top two values are within
  1e-5 of each other (then any of them);
* token: where float32 rounding can move a draw across a cumulative-mass
  boundary several tokens are correct, so the check is that the oracle's
  cumulative bounds of the returned token contain u up to 1e-4, and that the
  token is the oracle's own wherever u is farther than that from a boundary.

The one-call output head (dfa_output_head) is held to the same bars, below and
above 32768 tokens (one-launch and chunked mixture), up to 128256 tokens, with
128- and 64-row GEMV plans, sliced batches and a split-k plan; against the
two-call path every output is bit for bit the same.

Exact properties of the library's own outputs (bit for bit): the token is the
inverse-CDF token of the returned p_mix under the library's stated integer
masses (each value scaled by 2^35 and truncated; target = floor(u * total)),
and the greedy token is the first argmax of the returned p_mix.
"""
import numpy as np
import pytest
import torch

import dual_flow_shared_decode_amd as dfa
import workloads as W
from gpu_util import TOL, assert_close, say
from oracle import layer as LY
from oracle import mixture as MX
from workloads.device import to_device

pytestmark = pytest.mark.gpu

ALPHA_TOL = 5e-5
CDF_SLACK = 1e-4


def run_mixture(l1, l2, u, with_p_mix=True):
    b, v = l1.shape
    d = dfa.MixtureDesc(batch=b, vocab=v)
    ws = torch.full((dfa.dfa_mixture_workspace_size(d) // 4,), float("nan"), device="cuda")
    t1 = l1 if torch.is_tensor(l1) else to_device(np.ascontiguousarray(l1, dtype=np.float32))
    t2 = l2 if torch.is_tensor(l2) else to_device(np.ascontiguousarray(l2, dtype=np.float32))
    tu = to_device(np.ascontiguousarray(u, dtype=np.float32))
    tok = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    gr = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    al = torch.full((b,), float("nan"), device="cuda")
    pm = torch.full((b, v), float("nan"), device="cuda") if with_p_mix else None
    dfa.dfa_mixture_sample(d, t1, t2, tu, tok, gr, al, pm, ws)
    torch.cuda.synchronize()
    out = {"token": tok.cpu().numpy(), "greedy": gr.cpu().numpy(), "alpha": al.cpu().numpy()}
    if with_p_mix:
        out["p_mix"] = pm.cpu().numpy()
    return out


def fixed_point_token(p_mix, u):
    """Inverse-CDF token of float32 rows p_mix under integer masses floor(p * 2^35)."""
    m = (np.asarray(p_mix, dtype=np.float32) * np.float32(2.0 ** 35)).astype(np.uint64)
    cum = np.cumsum(m, axis=-1, dtype=np.uint64)
    total = cum[:, -1]
    uc = np.clip(np.asarray(u, dtype=np.float32), 0.0, np.float32(1.0 - 2.0 ** -24)).astype(np.float64)
    target = np.minimum((uc * total.astype(np.float64)).astype(np.uint64), total - np.uint64(1))
    return np.array([np.flatnonzero(cum[b] > target[b])[0] for b in range(len(uc))], dtype=np.int32)


def check_exact(got, u, what=""):
    assert np.array_equal(got["token"], fixed_point_token(got["p_mix"], u)), f"{what}: token vs its own p_mix"
    assert np.array_equal(got["greedy"], np.argmax(got["p_mix"], axis=-1)), f"{what}: greedy vs its own p_mix"


def check_against_oracle(got, l1, l2, u, what=""):
    u_eff = np.clip(np.asarray(u, dtype=np.float32), 0.0, np.float32(1.0 - 2.0 ** -24)).astype(np.float64)
    ref = MX.mixture(l1, l2, u_eff)
    b = len(u_eff)
    err_a = np.max(np.abs(got["alpha"] - ref["alpha"]))
    say(f"  {what}: alpha max abs err {err_a:.2e}")
    assert err_a <= ALPHA_TOL, f"{what}: alpha error {err_a}"
    if "p_mix" in got:
        assert_close(got["p_mix"], ref["p_mix"], TOL, f"{what} p_mix")
        check_exact(got, u, what)
    # greedy
    pm = ref["p_mix"]
    top2 = np.sort(pm, axis=-1)[:, -2:] if pm.shape[1] > 1 else np.repeat(pm, 2, axis=1)
    rows = np.arange(b)
    assert np.all((got["greedy"] >= 0) & (got["greedy"] < pm.shape[1])), f"{what}: greedy out of range"
    near_tie = (top2[:, 1] - top2[:, 0]) <= 1e-5 * top2[:, 1]
    ok_g = (got["greedy"] == ref["greedy"]) | (near_tie & (pm[rows, got["greedy"]] >= top2[:, 0]))
    assert np.all(ok_g), f"{what}: greedy {got['greedy'][~ok_g]} vs {ref['greedy'][~ok_g]}"
    # sampled token
    tok = got["token"]
    assert np.all((tok >= 0) & (tok < pm.shape[1])), f"{what}: token out of range"
    lo, hi = MX.cdf_bounds(pm, tok)
    ok = (lo - CDF_SLACK <= u_eff) & (u_eff < hi + CDF_SLACK)
    assert np.all(ok), f"{what}: token {tok[~ok]} bounds {lo[~ok]}..{hi[~ok]} u {u_eff[~ok]}"
    lo_o, hi_o = MX.cdf_bounds(pm, ref["token"])
    far = np.minimum(np.abs(u_eff - lo_o), np.abs(hi_o - u_eff)) > CDF_SLACK
    assert np.all(tok[far] == ref["token"][far]), f"{what}: tokens differ away from a boundary"
    say(f"  {what}: tokens equal to the oracle's: {int(np.sum(tok == ref['token']))}/{b}")
    return ref


@pytest.mark.parametrize("batch,vocab", [(3, 4), (1, 8), (2, 4096), (5, 4100), (4, 8192 + 4), (300, 1024),
                                         (3, 32768), (3, 32772), (4, 128256), (2, 152064), (1, 1 << 20)])
def test_mixture_matches_oracle(batch, vocab):
    cfg = W.MIX.replace(batch=batch, vocab=vocab)
    l1, l2, u = W.make_mixture_case(cfg, 11 + vocab)
    say(f"case mixture batch {batch} vocab {vocab}")
    check_against_oracle(run_mixture(l1, l2, u), l1, l2, u, f"b{batch} v{vocab}")


def test_mixture_full_workload():
    l1, l2, u = W.make_mixture_case(W.MIX, W.SEEDS["mix"])
    say("case mixture batch 32 vocab 32000")
    got = run_mixture(l1, l2, u)
    check_against_oracle(got, l1, l2, u, "mix")
    # without p_mix: the same decisions, bit for bit; and repeated calls agree
    bare = run_mixture(l1, l2, u, with_p_mix=False)
    again = run_mixture(l1, l2, u)
    for key in ("token", "greedy", "alpha"):
        assert np.array_equal(bare[key], got[key]), key
        assert np.array_equal(again[key], got[key]), key
    assert np.array_equal(again["p_mix"], got["p_mix"])


def test_u_edges():
    cfg = W.MIX.replace(batch=8, vocab=5000, peak_rows=0.0)
    l1, l2, _ = W.make_mixture_case(cfg, 21)
    u = np.array([0.0, 1.0, 1.0 - 2.0 ** -24, 0.5, -0.25, 2.0, 1e-30, 0.999], dtype=np.float32)
    say("case mixture u edges")
    got = run_mixture(l1, l2, u)
    check_against_oracle(got, l1, l2, u, "u edges")
    p = MX.mixture(l1, l2)["p_mix"]
    assert got["token"][0] == np.flatnonzero(p[0] > 0)[0] == 0  # u = 0: the first token with mass
    assert got["token"][4] == 0  # u < 0 clamps to 0
    assert got["token"][1] == got["token"][5]  # u >= 1 clamps to the same value


def test_degenerate_distributions():
    v = 4096 + 128
    rng = np.random.default_rng(5)
    base = rng.standard_normal((1, v)).astype(np.float32)
    flat = np.zeros((1, v), np.float32)
    peak = base.copy()
    peak[0, 123] = 100.0
    tie = base.copy()
    tie[0, [7, 3000]] = 20.0
    huge = (rng.standard_normal((1, v)) * 1e4).astype(np.float32)
    cases = {
        "equal flows": (base, base),
        "flat primary": (flat, base),
        "both flat": (flat, flat),
        "confident primary": (peak, base),
        "tied maxima": (tie, tie),
        "huge logits": (huge, -huge),
    }
    for name, (a, b) in cases.items():
        say(f"case mixture {name}")
        u = np.array([0.37], np.float32)
        got = run_mixture(a, b, u)
        ref = check_against_oracle(got, a, b, u, name)
        if name == "equal flows":
            assert_close(got["p_mix"], ref["p1"], TOL, "p_mix = p1")
        if name in ("flat primary", "both flat"):
            assert abs(got["alpha"][0] - 0.5 * (1 + 1.0 / v)) <= ALPHA_TOL
        if name == "both flat":
            assert got["greedy"][0] == 0 and got["token"][0] in (int(0.37 * v) - 1, int(0.37 * v), int(0.37 * v) + 1)
        if name == "confident primary":
            assert got["alpha"][0] >= 1 - 1e-6 and got["greedy"][0] == 123 and got["token"][0] == 123
        if name == "tied maxima":
            assert got["greedy"][0] == 7


def run_head(cfg, seed):
    """Dual output head: logits_f = h_f W^T from one read of W (dfa_dual_gemv), then the mixture."""
    h1, h2, w_bits, u = W.make_head_case(cfg, seed)
    wdev = to_device(w_bits)
    wt = torch.empty_like(wdev)
    dfa.dfa_pack_weight(wdev, wt, cfg.vocab, cfg.hidden)
    del wdev
    d = dfa.GemvDesc(batch=cfg.batch, n=cfg.vocab, k=cfg.hidden, num_flows=2, epilogue=dfa.DFA_EPI_NONE,
                     x_exact_bf16=1, k_split=0, rows_per_wg=0)
    ws = torch.empty(max(dfa.dfa_dual_gemv_workspace_size(d) // 4, 4), device="cuda")
    y1 = torch.empty((cfg.batch, cfg.vocab), device="cuda")
    y2 = torch.empty_like(y1)
    dfa.dfa_dual_gemv(d, wt, None, to_device(h1), to_device(h2), None, None, None, y1, y2, None, ws)
    got = run_mixture(y1, y2, u)
    logits = (y1.cpu().numpy(), y2.cpu().numpy())
    return h1, h2, w_bits, u, logits, got


@pytest.mark.parametrize("cfg", [W.HEAD.replace(batch=3, hidden=512, vocab=4096 + 64),
                                 W.HEAD.replace(batch=17, hidden=1024, vocab=8000), W.HEAD],
                         ids=["small", "ragged", "head"])
def test_dual_output_head(cfg):
    say(f"case output head batch {cfg.batch} hidden {cfg.hidden} vocab {cfg.vocab}")
    h1, h2, w_bits, u, (g1, g2), got = run_head(cfg, W.SEEDS["head"])
    r1, r2 = LY.linear(h1, w_bits), LY.linear(h2, w_bits)
    assert_close(g1, r1, TOL, "logits 1")
    assert_close(g2, r2, TOL, "logits 2")
    check_against_oracle(got, r1, r2, u, "head")


def run_fused_head(cfg, seed, with_p_mix=True):
    """dfa_output_head: both flows' logits and the mixture in one call."""
    h1, h2, w_bits, u = W.make_head_case(cfg, seed)
    wdev = to_device(w_bits)
    wt = torch.empty_like(wdev)
    dfa.dfa_pack_weight(wdev, wt, cfg.vocab, cfg.hidden)
    del wdev
    d = dfa.HeadDesc(batch=cfg.batch, vocab=cfg.vocab, hidden=cfg.hidden, x_exact_bf16=1)
    ws = torch.full((dfa.dfa_output_head_workspace_size(d) // 4,), float("nan"), device="cuda")
    b, v = cfg.batch, cfg.vocab
    y1 = torch.full((b, v), float("nan"), device="cuda")
    y2 = torch.full_like(y1, float("nan"))
    tok = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    gr = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    al = torch.full((b,), float("nan"), device="cuda")
    pm = torch.full((b, v), float("nan"), device="cuda") if with_p_mix else None
    dfa.dfa_output_head(d, wt, to_device(h1), to_device(h2), to_device(u), y1, y2, tok, gr, al, pm, ws)
    torch.cuda.synchronize()
    got = {"token": tok.cpu().numpy(), "greedy": gr.cpu().numpy(), "alpha": al.cpu().numpy()}
    if with_p_mix:
        got["p_mix"] = pm.cpu().numpy()
    return h1, h2, w_bits, u, (y1.cpu().numpy(), y2.cpu().numpy()), got


HEADS = {
    # up to 32768 tokens: the GEMV, then the one-launch mixture
    "head": W.HEAD,
    # above: the chunked mixture (64-row GEMV plan; 128-row plan; 32 chunks)
    "rows64": W.HEAD.replace(batch=3, hidden=512, vocab=40000),
    "rows128": W.HEAD.replace(batch=5, hidden=2048, vocab=40960),
    "vocab128k": W.HEAD.replace(batch=4, hidden=512, vocab=128256),
    # 40 sequences: the GEMV in slices of 32, the mixture over all 40
    "batch40": W.HEAD.replace(batch=40, hidden=2048, vocab=40960),
    # a plan that splits k (too few row groups): GEMV, reduction, then the mixture's own kernels
    "split": W.HEAD.replace(batch=3, hidden=512, vocab=4096 + 64),
}


@pytest.mark.parametrize("name", list(HEADS))
def test_fused_output_head(name):
    cfg = HEADS[name]
    say(f"case fused output head {name}: batch {cfg.batch} hidden {cfg.hidden} vocab {cfg.vocab}")
    h1, h2, w_bits, u, (g1, g2), got = run_fused_head(cfg, W.SEEDS["head"])
    r1, r2 = LY.linear(h1, w_bits), LY.linear(h2, w_bits)
    assert_close(g1, r1, TOL, "logits 1")
    assert_close(g2, r2, TOL, "logits 2")
    check_against_oracle(got, r1, r2, u, name)
    # without p_mix: the same tokens and alpha
    *_, got2 = run_fused_head(cfg, W.SEEDS["head"], with_p_mix=False)
    for k in ("token", "greedy", "alpha"):
        assert np.array_equal(got2[k], got[k]), k


@pytest.mark.parametrize("vocab", [32000, 40960])
def test_fused_head_matches_the_two_call_path(vocab):
    """dfa_output_head and dfa_dual_gemv + dfa_mixture_sample: every output bit for bit the same."""
    cfg = W.HEAD.replace(batch=8, hidden=2048, vocab=vocab)
    say(f"case one-call head vs two calls, vocab {vocab}")
    *_, (f1, f2), fused = run_fused_head(cfg, 91)
    *_, (t1, t2), two = run_head(cfg, 91)
    assert np.array_equal(f1, t1) and np.array_equal(f2, t2)
    for k in ("token", "greedy", "alpha", "p_mix"):
        assert np.array_equal(fused[k], two[k]), k


@pytest.mark.parametrize("vocab", [32000, 40000])
def test_non_finite_rows_return_the_defined_token(vocab):
    """A row with a non-finite logit has no finite mixture mass: both paths (one launch up to
    32768 tokens, chunked above) return token and greedy vocab - 1 for it, never an index
    outside the vocabulary, and the other rows are untouched (regression: the chunked pick
    once read an unset chunk index for such a row)."""
    cfg = W.MIX.replace(batch=5, vocab=vocab)
    l1, l2, u = W.make_mixture_case(cfg, 71 + vocab)
    l1 = l1.copy()
    l2 = l2.copy()
    l1[1, 17] = np.nan          # primary NaN
    l2[3, vocab - 5] = np.nan   # auxiliary NaN
    l1[4, 123] = np.inf         # primary +inf
    bad = np.array([1, 3, 4])
    good = np.array([0, 2])
    say(f"case mixture non-finite rows, vocab {vocab}")
    got = run_mixture(l1, l2, u)
    assert np.all(got["token"][bad] == vocab - 1), got["token"]
    assert np.all(got["greedy"][bad] == vocab - 1), got["greedy"]
    sub = {k: v[good] for k, v in got.items()}
    check_against_oracle(sub, l1[good], l2[good], u[good], f"finite rows v{vocab}")
