"""Pins of oracle.mixture against brute force, library routines, closed forms and invariants.

The mixture is p_mix = alpha p1 + (1 - alpha) p2 with alpha = (1 + sum p1^2) / 2
(the reading of [DFT-pt] "Mecanismos Chave" stated in oracle/mixture.py); a
draw u picks the smallest token whose cumulative mass exceeds u.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import mixture as MX


def brute_mixture(l1, l2, u):
    """Scalar loops with math.exp / math.fsum, independent of the oracle's numpy code."""
    out = []
    for row1, row2, ub in zip(l1.tolist(), l2.tolist(), u.tolist()):
        m1, m2 = max(row1), max(row2)
        e1 = [math.exp(x - m1) for x in row1]
        e2 = [math.exp(x - m2) for x in row2]
        s1, s2 = math.fsum(e1), math.fsum(e2)
        p1 = [x / s1 for x in e1]
        p2 = [x / s2 for x in e2]
        c = math.fsum(x * x for x in p1)
        a = 0.5 + 0.5 * c
        pm = [a * x + (1 - a) * y for x, y in zip(p1, p2)]
        total, run, tok = math.fsum(pm), 0.0, len(pm) - 1
        for v, x in enumerate(pm):
            run += x
            if run > ub * total:
                tok = v
                break
        best = max(range(len(pm)), key=lambda v: (pm[v], -v))
        out.append((a, pm, tok, best))
    return out


def rand_case(seed, b=4, v=11, scale=2.0):
    rng = np.random.default_rng(seed)
    l1 = (rng.standard_normal((b, v)) * scale).astype(np.float32)
    l2 = (rng.standard_normal((b, v)) * scale).astype(np.float32)
    u = rng.random(b)
    return l1, l2, u


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force(seed):
    l1, l2, u = rand_case(seed)
    got = MX.mixture(l1, l2, u)
    for b, (a, pm, tok, best) in enumerate(brute_mixture(l1, l2, u)):
        assert abs(got["alpha"][b] - a) <= 1e-12
        assert np.max(np.abs(got["p_mix"][b] - np.array(pm))) <= 1e-12
        assert got["token"][b] == tok
        assert got["greedy"][b] == best


def test_softmax_and_sampling_match_library_routines():
    l1, l2, u = rand_case(3, b=6, v=50)
    got = MX.mixture(l1, l2, u)
    assert np.max(np.abs(got["p1"] - scipy.special.softmax(l1.astype(np.float64), axis=-1))) <= 1e-12
    assert np.max(np.abs(got["p2"] - scipy.special.softmax(l2.astype(np.float64), axis=-1))) <= 1e-12
    for b in range(6):
        cdf = np.cumsum(got["p_mix"][b])
        assert got["token"][b] == np.searchsorted(cdf, u[b] * cdf[-1], side="right")


def test_closed_forms():
    v = 8
    flat = np.zeros((1, v), np.float32)
    other = np.arange(v, dtype=np.float32)[None]
    got = MX.mixture(flat, other)
    assert abs(got["collision"][0] - 1.0 / v) <= 1e-15
    assert abs(got["alpha"][0] - 0.5 * (1 + 1.0 / v)) <= 1e-15
    # a dominant primary logit: collision 1, alpha 1, the mixture is the primary distribution
    peak = np.zeros((1, v), np.float32)
    peak[0, 3] = 1000.0
    got = MX.mixture(peak, other)
    assert got["alpha"][0] == 1.0 and np.array_equal(got["p_mix"], got["p1"])
    # two tokens: p1 = (sigmoid(x), 1 - sigmoid(x))
    x = 1.3
    got = MX.mixture(np.array([[x, 0.0]], np.float32), np.array([[0.0, 0.0]], np.float32))
    s = 1.0 / (1.0 + math.exp(-float(np.float32(x))))
    c = s * s + (1 - s) * (1 - s)
    assert abs(got["alpha"][0] - (1 + c) / 2) <= 1e-14
    a = (1 + c) / 2
    assert abs(got["p_mix"][0, 0] - (a * s + (1 - a) * 0.5)) <= 1e-14


def test_invariants():
    l1, l2, u = rand_case(4, b=5, v=40)
    got = MX.mixture(l1, l2, u)
    assert np.max(np.abs(got["p_mix"].sum(-1) - 1)) <= 1e-12
    assert np.all(got["alpha"] >= 0.5) and np.all(got["alpha"] <= 1.0)
    # alpha depends on the primary alone
    assert np.array_equal(MX.mixture(l1, -l2)["alpha"], got["alpha"])
    # equal flows: the mixture is their distribution
    same = MX.mixture(l1, l1)
    assert np.max(np.abs(same["p_mix"] - same["p1"])) <= 1e-15
    # a constant added to a flow's logits changes nothing
    shifted = MX.mixture(l1.astype(np.float64) + 3.0, l2.astype(np.float64) - 5.0, u)
    assert np.max(np.abs(shifted["p_mix"] - got["p_mix"])) <= 1e-12
    # relabelling the vocabulary relabels the mixture
    perm = np.random.default_rng(0).permutation(40)
    permuted = MX.mixture(l1[:, perm], l2[:, perm])
    assert np.max(np.abs(permuted["p_mix"] - got["p_mix"][:, perm])) <= 1e-15
    assert np.max(np.abs(permuted["alpha"] - got["alpha"])) <= 1e-15


def test_sampling_properties():
    l1, l2, _ = rand_case(5, b=2, v=30)
    p = MX.mixture(l1, l2)["p_mix"]
    n = 4000
    us = (np.arange(n) + 0.5) / n
    toks = np.stack([MX.sample(p, np.full(2, x)) for x in us])  # [n, 2]
    assert np.all(np.diff(toks, axis=0) >= 0)  # monotone in u
    assert np.all(MX.sample(p, np.zeros(2)) == 0)  # every token has mass here
    for b in range(2):
        lo, hi = MX.cdf_bounds(p[b:b + 1].repeat(n, 0), toks[:, b])
        assert np.all(lo <= us + 1e-15) and np.all(us < hi + 1e-15)
        counts = np.bincount(toks[:, b], minlength=30)
        assert np.all(np.abs(counts - n * p[b] / p[b].sum()) <= 1.0 + 1e-9)  # stratified draws


@pytest.mark.parametrize("mistake", ["alpha_from_aux", "no_floor", "swapped", "alpha_from_max"])
def test_planted_mistake_is_caught(mistake, monkeypatch):
    """A plausible error planted in the oracle fails at least one pin above."""
    real = MX.mixture

    def planted(l1, l2, u=None):
        out = real(l1, l2, u)
        p1, p2 = out["p1"], out["p2"]
        if mistake == "alpha_from_aux":
            a = 0.5 * (1 + (p2 * p2).sum(-1))
        elif mistake == "no_floor":
            a = (p1 * p1).sum(-1)
        elif mistake == "swapped":
            a = out["alpha"]
            out["p_mix"] = (1 - a)[:, None] * p1 + a[:, None] * p2
            return out
        else:
            a = 0.5 * (1 + p1.max(-1))
        out["alpha"] = a
        out["p_mix"] = a[:, None] * p1 + (1 - a)[:, None] * p2
        return out

    monkeypatch.setattr(MX, "mixture", planted)
    checks = [test_matches_brute_force, test_closed_forms, test_invariants]
    failed = 0
    for check in checks:
        try:
            check(0) if check is test_matches_brute_force else check()
        except AssertionError:
            failed += 1
    assert failed >= 1
