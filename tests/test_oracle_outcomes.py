"""Pins of the oracle's outcome scoring and cache selection against what the
pages and the mathematics fix.  CPU only.

JetSpec++, Section 4.2 ("Outcome Selection") and Appendix F.1: from the
decoder's rows p(.|j), j = 0..gamma, and the block's draft tokens, the score
of outcome (k, a) is P(k, a) = prod_{i<k} p_i(x_i) * p_k(a) (a != x_k for
k < gamma); by Proposition 1 this is exactly the probability that
point-mass verification ends at (k, a).  The cache keeps the B most probable
outcomes and its hit probability is their sum.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from enumerate_law import outcome_law

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def logp(p):
    with np.errstate(divide="ignore"):
        return f32(np.log(np.asarray(p, dtype=np.float64)))


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("T", [0.6, 1.0])
def test_scores_equal_point_mass_verification_law(seed, T):
    """Proposition 1: the scores are the exact law of the verification outcome,
    here found by bisecting the point-mass verification oracle's decision
    boundaries (an independent computation)."""
    rng = np.random.default_rng(300 + seed)
    V, g = 5, 3
    z = f32(rng.normal(0, 1.4, (g + 1, V)))
    d = rng.integers(0, V, g).astype(np.int32)
    law, _ = outcome_law(z, np.zeros((g, V), np.float32), d, T=T, rule="pointmass")
    r = oracle.outcome_topk(z[None], d[None], T, ncache=4, want_all=True)
    P = r["all_scores"][0]
    for k in range(g + 1):
        for a in range(V):
            assert abs(P[k, a] - law.get((k, a), 0.0)) < 1e-13, (k, a)
    assert abs(P.sum() - 1.0) < 1e-13  # disjoint, exhaustive outcomes


def test_worked_example_024():
    """JetSpec++ Appendix F.1: P(1, b) = p_1 * p(b | 1) = 0.8 * 0.3 = 0.24."""
    with open(os.path.join(GOLD, "worked_example_f1.json")) as f:
        g = json.load(f)
    p1 = [g["p1"]["d1"], g["p1"]["other"] / 2, g["p1"]["other"] / 2]
    p2 = [g["p2"]["d2"], g["p2"]["b"], g["p2"]["rest"]]
    z = np.stack([logp(p1), logp(p2), logp([0.2, 0.3, 0.5])])
    r = oracle.outcome_topk(z[None], np.array([[0, 0]]), 1.0, ncache=3, want_all=True)
    assert abs(r["all_scores"][0, 1, 1] - g["p_end_at_1_b"]) < 1e-7
    # the rejected draft token is not an outcome at its position
    assert r["all_scores"][0, 0, 0] == 0.0 and r["all_scores"][0, 1, 0] == 0.0


@pytest.mark.parametrize("seed", range(20))
def test_cache_maximises_hit_probability(seed):
    """A block ends in exactly one outcome, so a cache's chance of holding the
    realised one adds up over its entries, and no B-subset beats the B
    largest scores: checked by brute force over every B-subset of a tiny
    block ("JetSpec++", Section 4.2 "Outcome Selection")."""
    rng = np.random.default_rng(400 + seed)
    V, g, B = 3, 2, 3
    z = f32(rng.normal(0, 1.0, (g + 1, V)))
    d = rng.integers(0, V, g).astype(np.int32)
    r = oracle.outcome_topk(z[None], d[None], 1.0, ncache=B, want_all=True)
    P = r["all_scores"][0]
    outcomes = [(k, a) for k in range(g + 1) for a in range(V) if k == g or a != d[k]]
    best = max(sum(P[k, a] for k, a in sub) for sub in itertools.combinations(outcomes, B))
    assert abs(r["hit"][0] - best) < 1e-15
    assert abs(r["hit"][0] - r["p"][0].sum()) < 1e-15
    # the kept entries are listed from most to least probable, and are outcomes
    assert (np.diff(r["p"][0]) <= 0).all()
    for k, a in zip(r["k"][0], r["a"][0]):
        assert (int(k), int(a)) in outcomes


def test_fewer_outcomes_than_slots_and_ties():
    """Zero-probability outcomes (masked tokens) are never kept; slots beyond
    the positive outcomes hold -1; equal scores go to the smaller k, then the
    smaller token."""
    z = np.full((1, 2, 4), -np.inf, np.float32)
    z[0, 0, [0, 2]] = 0.0  # p_0 = (1/2, 0, 1/2, 0)
    z[0, 1, [1, 3]] = 0.0  # p_1 = (0, 1/2, 0, 1/2)
    r = oracle.outcome_topk(z, np.array([[0]]), 1.0, ncache=6)
    # outcomes: (0, 2) = 1/2, (1, 1) = (1, 3) = 1/4
    assert r["k"][0].tolist() == [0, 1, 1, -1, -1, -1]
    assert r["a"][0].tolist() == [2, 1, 3, -1, -1, -1]
    assert np.allclose(r["p"][0], [0.5, 0.25, 0.25, 0, 0, 0])
    assert r["hit"][0] == 1.0


def test_invalid_request_flagged_alone():
    rng = np.random.default_rng(9)
    z = f32(rng.normal(0, 1, (3, 3, 10)))
    d = rng.integers(0, 10, (3, 2)).astype(np.int32)
    d[1, 1] = 10
    r = oracle.outcome_topk(z, d, 1.0, ncache=4)
    assert r["hit"][1] == -1.0 and (r["k"][1] == -1).all() and (r["a"][1] == -1).all()
    assert (r["hit"][[0, 2]] > 0).all()


def test_hit_probability_grows_with_cache_size():
    rng = np.random.default_rng(10)
    z = f32(rng.normal(0, 2.0, (4, 9, 500)))
    d = rng.integers(0, 500, (4, 8)).astype(np.int32)
    prev = np.zeros(4)
    for B in (1, 2, 4, 8, 16):
        h = oracle.outcome_topk(z, d, 0.8, ncache=B)["hit"]
        assert (h >= prev - 1e-15).all() and (h <= 1 + 1e-12).all()
        prev = h


@pytest.mark.parametrize("seed", range(3))
def test_lookup_hit_rate_is_the_cache_hit_probability(seed):
    """Sampling the point-mass verification of one block many times and
    looking each outcome up in the block's cache hits slot c with probability
    p_c, and some slot with the cache's hit probability (Proposition 1: the
    verified outcome has law P(k, a)).  Three oracle functions are checked
    against each other; N = 40000 draws, bounds of 5 standard deviations."""
    rng = np.random.default_rng(500 + seed)
    V, g, B, N = 40, 3, 6, 40000
    z = f32(rng.normal(0, 1.5, (g + 1, V)))
    z[:, 0] += 2.0  # a likely draft token
    d = np.zeros(g, np.int32)
    cache = oracle.outcome_topk(z[None], d[None], 0.8, ncache=B)
    u = rng.random((N, g + 1), dtype=np.float32)
    ver = oracle.chain_pointmass(np.broadcast_to(z, (N, g + 1, V)).copy(),
                                 np.broadcast_to(d, (N, g)).copy(), u, 0.8)
    slot = oracle.cache_lookup(ver["accept_len"], ver["out_tokens"],
                               np.broadcast_to(cache["k"], (N, B)), np.broadcast_to(cache["a"], (N, B)))
    h = cache["hit"][0]
    assert abs((slot >= 0).mean() - h) < 5 * np.sqrt(h * (1 - h) / N)
    for c in range(B):
        pc = cache["p"][0, c]
        assert abs((slot == c).mean() - pc) < 5 * np.sqrt(pc * (1 - pc) / N) + 1e-12, c


def test_lookup_cases():
    """Definition cases: the first matching slot wins, unused slots (-1) and
    invalid blocks never match, and a is the token after the k accepted ones."""
    acc = np.array([2, 0, -1, 3], np.int32)
    out = np.array([[5, 6, 7, -1], [9, -1, -1, -1], [-1, -1, -1, -1], [1, 2, 3, 4]], np.int32)
    ck = np.array([[2, 2, -1], [0, 1, -1], [-1, -1, -1], [3, 3, 0]], np.int32)
    ca = np.array([[6, 7, -1], [9, 9, -1], [-1, -1, -1], [3, 4, 4]], np.int32)
    assert oracle.cache_lookup(acc, out, ck, ca).tolist() == [1, 0, -1, 1]
