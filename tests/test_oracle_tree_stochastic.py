"""Pins of the oracle's stochastic tree verification against what the pages
and the mathematics fix.  CPU only.

"JetSpec" reading notes, section "Tree verification": every drafted token is
tested with a Bernoulli of probability alpha = min(1, p/q) (Eq. 16), a
branch keeps its longest accepted prefix (Eq. 17), the best branch is the
deepest accepted one, and the correction token is sampled from the target
after it (Fig. 5).  The tests drive the oracle with uniforms placed inside
each decision's interval, so every outcome is fixed and is predicted here
from an independent computation of the probabilities.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import log_softmax, softmax

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def random_tree(rng, n, max_children=3):
    par = [-1]
    kids = [0]
    for j in range(1, n):
        cand = [i for i in range(j) if kids[i] < max_children]
        p = int(rng.choice(cand))
        par.append(p)
        kids[p] += 1
        kids.append(0)
    return np.array(par, np.int32)


def predict(tgt, drf, par, tok, T, pattern, draw_rank, rng):
    """Uniforms that realise a pass/fail pattern, and the outcome they must
    give, from scipy's softmax (independent of the oracle)."""
    n, V = tgt.shape
    lp = log_softmax(tgt.astype(np.float64) / T, axis=1)
    lq = log_softmax(drf.astype(np.float64) / T, axis=1)
    u = np.zeros(n, np.float32)
    acc = np.zeros(n, bool)
    acc[0] = True
    depth = np.zeros(n, int)
    for j in range(1, n):
        p, y = par[j], tok[j]
        a = 1.0 if lq[p, y] == -np.inf and lp[p, y] > -np.inf else min(1.0, np.exp(lp[p, y] - lq[p, y]))
        passes = pattern[j] if 0.0 < a < 1.0 else a == 1.0
        u[j] = a * 0.5 if passes else (1.0 + a) * 0.5
        acc[j] = acc[p] and passes
        depth[j] = depth[p] + 1
    best = max((j for j in range(n) if acc[j]), key=lambda j: (depth[j], -j))
    pb = softmax(tgt[best].astype(np.float64) / T)
    pos = np.nonzero(pb > 1e-6)[0]
    t = int(pos[draw_rank % len(pos)])
    c = np.cumsum(pb)
    u[0] = (c[t] - pb[t] * 0.5) / c[-1]
    path = []
    j = best
    while j != 0:
        path.append(int(tok[j]))
        j = par[j]
    return u, depth[best], best, path[::-1] + [t], pb


@pytest.mark.parametrize("seed", range(30))
def test_fixed_outcomes_from_independent_probabilities(seed):
    rng = np.random.default_rng(900 + seed)
    n, V, T = int(rng.integers(2, 12)), int(rng.integers(3, 40)), float(rng.choice([0.6, 1.0, 1.7]))
    tgt = f32(rng.normal(0, 1.5, (n, V)))
    drf = f32(tgt + rng.normal(0, 0.8, (n, V)))
    par = random_tree(rng, n)
    tok = rng.integers(0, V, n).astype(np.int32)
    # half of the tokens are the target's most likely ones, so paths get long
    for j in range(1, n):
        if rng.random() < 0.5:
            tok[j] = int(np.argmax(tgt[par[j]]))
    pattern = rng.random(n) < 0.7
    u, k, best, out, pb = predict(tgt, drf, par, tok, T, pattern, int(rng.integers(0, 99)), rng)
    r = oracle.tree_stochastic(tgt[None], drf[None], par[None], tok[None], u[None], T,
                               dtype="f32", want_dist=True)
    assert r["accept_len"][0] == k and r["accept_node"][0] == best
    assert r["out_tokens"][0, :k + 1].tolist() == out
    assert (r["out_tokens"][0, k + 1:] == -1).all()
    assert np.abs(r["final_dist"][0] - pb).max() < 1e-12  # the correction law: p after the path


def test_figure5_worked_example():
    """[JN] Fig. 5: are/told/that accepted, given and sum rejected; the best
    branch 'are told that' (a = 3) then the correction ':' -- 4 tokens.  The
    target rows are one-hot on the figure's next words, so every test is
    certain (alpha is 1 for the target's word, 0 otherwise) whatever the
    draft rows and the uniforms."""
    with open(os.path.join(GOLD, "fig5_tree.json")) as f:
        g = json.load(f)
    vocab = {w: i for i, w in enumerate(g["vocab"])}
    n, V = len(g["nodes"]), len(vocab)
    tgt = np.full((n, V), -np.inf, np.float32)
    par = np.zeros(n, np.int32)
    tok = np.zeros(n, np.int32)
    for nd in g["nodes"]:
        tgt[nd["id"], vocab[nd["target_argmax"]]] = 0.0
        par[nd["id"]] = nd["parent"]
        tok[nd["id"]] = vocab[nd["token"]]
    rng = np.random.default_rng(5)
    drf = f32(rng.normal(0, 1, (n, V)))
    u = rng.random(n).astype(np.float32)
    r = oracle.tree_stochastic(tgt[None], drf[None], par[None], tok[None], u[None], 1.0, dtype="f32")
    k = int(r["accept_len"][0])
    assert k == g["expected_accept_len"]
    assert [g["vocab"][t] for t in r["out_tokens"][0, :k]] == g["expected_path"]
    assert g["vocab"][r["out_tokens"][0, k]] == g["expected_bonus"]
    assert k + 1 == g["expected_committed"]


@pytest.mark.parametrize("seed", range(10))
def test_one_hot_target_is_greedy_verification(seed):
    """With one-hot target rows, alpha is 1 exactly when a token is the
    target's argmax and 0 otherwise, and p has all its mass there: the rule
    becomes greedy tree verification (a cross-check of two oracle functions
    on random trees with ties between siblings)."""
    rng = np.random.default_rng(950 + seed)
    B, n, V = 8, 40, 30
    d = synth.tree_inputs(B, n, V, seed=seed)
    amax = np.argmax(synth.bf16_to_f32(d["target"]), axis=2)
    tgt = np.full((B, n, V), -np.inf, np.float32)
    np.put_along_axis(tgt, amax[..., None], 0.0, axis=2)
    drf = f32(rng.normal(0, 1, (B, n, V)))
    u = rng.random((B, n)).astype(np.float32)
    s = oracle.tree_stochastic(synth.bf16_bits(tgt), synth.bf16_bits(drf), d["parents"], d["tokens"],
                               u, 0.8)
    gr = oracle.tree_greedy(synth.bf16_bits(tgt), d["parents"], d["tokens"])
    assert np.array_equal(s["accept_len"], gr["accept_len"])
    assert np.array_equal(s["accept_node"], gr["accept_node"])
    assert np.array_equal(s["out_tokens"], gr["out_tokens"])


def test_invalid_requests_flagged_alone():
    rng = np.random.default_rng(7)
    B, n, V = 5, 6, 12
    tgt = f32(rng.normal(0, 1, (B, n, V)))
    drf = f32(rng.normal(0, 1, (B, n, V)))
    par = np.tile(np.array([-1, 0, 0, 1, 2, 2], np.int32), (B, 1))
    tok = rng.integers(0, V, (B, n)).astype(np.int32)
    u = rng.random((B, n)).astype(np.float32)
    par[1, 3] = 3      # a parent that does not precede its child
    tok[2, 4] = V      # a token out of range
    drf[3, 1, 2] = np.nan
    tgt[4, 5, :] = -np.inf
    r = oracle.tree_stochastic(tgt, drf, par, tok, u, 1.0, dtype="f32")
    assert r["accept_len"].tolist()[1:] == [-1, -1, -1, -1] and r["accept_len"][0] >= 0
    assert (r["out_tokens"][1:] == -1).all() and (r["accept_node"][1:] == -1).all()


def test_masked_tokens():
    """A token the target gives probability 0 is always rejected; one the
    draft gives probability 0 (but the target does not) is always accepted."""
    V = 6
    tgt = np.zeros((3, V), np.float32)
    drf = np.zeros((3, V), np.float32)
    tgt[0, 2] = -np.inf
    drf[0, 4] = -np.inf
    par = np.array([-1, 0, 0], np.int32)
    tok = np.array([0, 2, 4], np.int32)
    u = np.array([0.5, 0.0, 0.999], np.float32)
    r = oracle.tree_stochastic(tgt[None], drf[None], par[None], tok[None], u[None], 1.0, dtype="f32")
    assert r["accept_len"][0] == 1 and r["accept_node"][0] == 2
