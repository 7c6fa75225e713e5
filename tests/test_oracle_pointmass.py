"""Pins of the oracle's point-mass ("exact-match") chain verification against
what the pages and the mathematics fix.  CPU only.

JetSpec++, Appendix F.3: with a point-mass proposal the draft offers each
token with certainty, so position i accepts with probability p_i(x_i); the
first rejection at k draws from p_k with x_k removed and renormalised; a
fully accepted block draws the bonus token from p_gamma.  The oracle is
driven as a black box of its uniforms (tests/enumerate_law.py bisects every
decision boundary), and the exact outcome law is compared with the worked
example of Appendix F.1, Proposition 1 and the closed form for the expected
number of committed tokens.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from enumerate_law import outcome_law

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def logp(p):
    with np.errstate(divide="ignore"):
        return f32(np.log(np.asarray(p, dtype=np.float64)))


def probs(z, T=1.0):
    return softmax(np.asarray(z, dtype=np.float64) / T)


def law_pm(tgt, d, T=1.0):
    g = len(d)
    V = tgt.shape[1]
    dummy = np.zeros((g, V), dtype=np.float32)  # the point-mass rule reads no draft logits
    return outcome_law(tgt, dummy, d, T=T, rule="pointmass")


def test_worked_example_024():
    """JetSpec++ Appendix F.1: P(end at (1, b)) = 0.8 * 0.5 * 0.6 = 0.24."""
    g = gold("worked_example_f1.json")
    p1 = [g["p1"]["d1"], g["p1"]["other"] / 2, g["p1"]["other"] / 2]
    p2 = [g["p2"]["d2"], g["p2"]["b"], g["p2"]["rest"]]
    tgt = np.stack([logp(p1), logp(p2), logp([0.2, 0.3, 0.5])])
    law, t = law_pm(tgt, [0, 0])
    assert abs(t[0] - g["p_accept_d1"]) < 1e-7
    assert abs((1 - t[1]) - g["p_reject_d2"]) < 1e-7
    assert abs(law[(1, 1)] - g["p_end_at_1_b"]) < 1e-7
    P1, P2 = probs(tgt[0]), probs(tgt[1])
    assert abs(law[(1, 1)] - P1[0] * P2[1]) < 1e-15
    assert (1, 0) not in law  # the rejected draft token is never the correction


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("T", [0.7, 1.0])
def test_proposition1_law(seed, T):
    """JetSpec++ Proposition 1: P(k, a) = prod_{j<k} p_j(x_j) * p_k(a) for
    a != x_k (k < gamma) and P(gamma, a) = prod_j p_j(x_j) * p_gamma(a)."""
    rng = np.random.default_rng(200 + seed)
    V, g = 5, 3
    tgt = f32(rng.normal(0, 1.3, (g + 1, V)))
    d = rng.integers(0, V, g)
    law, _ = law_pm(tgt, d, T=T)
    P = [probs(tgt[j], T) for j in range(g + 1)]
    want, run = {}, 1.0
    for k in range(g + 1):
        for a in range(V):
            if k < g and a == d[k]:
                continue
            want[(k, a)] = run * P[k][a]
        if k < g:
            run *= P[k][d[k]]
    for key in set(want) | set(law):
        assert abs(law.get(key, 0.0) - want.get(key, 0.0)) < 1e-14, key
    assert abs(sum(law.values()) - 1.0) < 1e-14


def test_expected_tokens_closed_form():
    """JetSpec reading notes, Eq. 2: with p_i(x_i) = alpha at every position,
    E[#committed tokens] = E[k + 1] = (1 - alpha^(gamma+1)) / (1 - alpha)."""
    alpha, g, V = 0.75, 4, 3
    p = [alpha, (1 - alpha) / 2, (1 - alpha) / 2]
    tgt = np.stack([logp(p)] * (g + 1))
    law, _ = law_pm(tgt, [0] * g)
    ek = sum((k + 1) * pr for (k, _a), pr in law.items())
    want = (1 - alpha ** (g + 1)) / (1 - alpha)
    alpha32 = probs(tgt[0])[0]  # the exactly decoded float32 logits
    want32 = (1 - alpha32 ** (g + 1)) / (1 - alpha32)
    assert abs(ek - want32) < 1e-12
    assert abs(ek - want) < 1e-6


def test_same_outcomes_as_ratio_test_with_one_hot_draft():
    """A one-hot draft row makes the ratio test min(1, p/q) equal to p(x) and
    the residual max(0, p - q) equal to p without x: both rules then give the
    same outcome for every uniform (a cross-check of two oracle functions)."""
    rng = np.random.default_rng(7)
    B, g, V = 200, 4, 37
    tgt = f32(rng.normal(0, 2.0, (B, g + 1, V)))
    d = rng.integers(0, V, (B, g)).astype(np.int32)
    drf = np.full((B, g, V), -np.inf, dtype=np.float32)
    for b in range(B):
        drf[b, np.arange(g), d[b]] = 0.0
    u = rng.random((B, g + 1), dtype=np.float32)
    a = oracle.chain(tgt, drf, d, u, 0.9, want_dist=True)
    pm = oracle.chain_pointmass(tgt, d, u, 0.9, want_dist=True)
    assert np.array_equal(a["accept_len"], pm["accept_len"])
    assert np.array_equal(a["out_tokens"], pm["out_tokens"])
    assert np.abs(a["final_dist"] - pm["final_dist"]).max() < 1e-12


def test_edge_cases():
    V, g = 6, 2
    # all target mass on the draft tokens: every test passes
    z = np.full((1, g + 1, V), -np.inf, dtype=np.float32)
    z[0, 0, 2] = 0.0
    z[0, 1, 4] = 0.0
    z[0, 2, :] = 0.0
    u = np.array([[0.999, 0.999, 0.6]], dtype=np.float32)  # C(3) = 4/6 is the first CDF value above 0.6
    r = oracle.chain_pointmass(z, np.array([[2, 4]]), u, 1.0)
    assert r["accept_len"][0] == 2 and r["out_tokens"][0].tolist() == [2, 4, 3]
    # a masked draft token (p = 0) is always rejected; the draw avoids it
    z = f32(np.random.default_rng(1).normal(0, 1, (1, g + 1, V)))
    z[0, 0, 3] = -np.inf
    u = np.array([[0.0, 0.0, 0.999]], dtype=np.float32)
    r = oracle.chain_pointmass(z, np.array([[3, 1]]), u, 1.0, want_dist=True)
    assert r["accept_len"][0] == 0 and r["out_tokens"][0, 0] != 3
    assert r["final_dist"][0, 3] == 0.0
    # a token out of range makes the block invalid
    r = oracle.chain_pointmass(z, np.array([[3, V]]), u, 1.0)
    assert r["accept_len"][0] == -1 and (r["out_tokens"][0] == -1).all()
