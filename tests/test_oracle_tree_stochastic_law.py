"""The law of the first committed token under the stochastic tree rule that
the library implements ("JetSpec" reading notes, section "Tree
verification": one Bernoulli test per node with probability min(1, p/q),
Eq. 16; the deepest fully accepted node wins, Eq. 17; the correction is drawn
from p after it, Fig. 5), found by exact enumeration of the oracle.  CPU
only.

Setting: the root has m children whose tokens are drawn independently from
the draft distribution q at the root; p is the target distribution at the
root.  Every child has depth 1, so v* is the lowest-index accepted child, or
the root when all are rejected.  With beta = sum_v min(p(v), q(v)) (the
probability that one child passes), each child is accepted with probability
beta independently, and an accepted child's token is distributed as
min(p, q) / beta.  Hence

    P(first token = y) = min(p, q)(y) * (1 - (1 - beta)^m) / beta
                         + (1 - beta)^m * p(y).

This is p only when beta = 1 (q = p): a rejected child leaves its token's
mass in p instead of removing it, as the residual max(0, p - q) does in
chain verification ("Speculative decoding verifies draft tokens ...",
section "Rejection uses a residual distribution").  For m = 1, p = (0.5,
0.5) and q = (0.9, 0.1): beta = 0.6, and token 0 is committed with
probability 0.5 + 0.4 * 0.5 = 0.7 instead of 0.5.

The enumeration treats the oracle as a black box: each test's acceptance
threshold is bisected on its uniform, every draft draw (all token tuples,
weighted by q) and every pass/fail pattern (weighted by the bisected
interval lengths) is run, and the draw after the pattern is read from the
oracle's final_dist.
"""
import itertools

import numpy as np
import pytest

import oracle

STEPS = 60


def f32(x):
    return np.asarray(x, dtype=np.float32)


def run(zp, zq, toks, u, want_dist=False):
    """One request: root row (zp, zq), children with tokens toks; the node
    rows after the children are copies of the root rows (they are never
    read: no node below depth 1 exists)."""
    m = len(toks)
    n = m + 1
    V = zp.shape[0]
    tgt = np.broadcast_to(zp, (n, V)).copy()[None]
    drf = np.broadcast_to(zq, (n, V)).copy()[None]
    par = np.array([[-1] + [0] * m], np.int32)
    tok = np.array([[0] + list(toks)], np.int32)
    return oracle.tree_stochastic(tgt, drf, par, tok, np.asarray(u, np.float64)[None], 1.0,
                                  dtype="f32", want_dist=want_dist)


def threshold(zp, zq, y):
    """sup{u : a single child with token y passes}, by bisection."""
    lo, hi = 0.0, 1.0
    if run(zp, zq, [y], [0.5, 0.0])["accept_node"][0] != 1:
        return 0.0
    for _ in range(STEPS):
        mid = 0.5 * (lo + hi)
        if run(zp, zq, [y], [0.5, mid])["accept_node"][0] == 1:
            lo = mid
        else:
            hi = mid
    return hi


def first_token_law(zp, zq, m):
    V = zp.shape[0]
    q = np.exp(zq.astype(np.float64) - zq.max())
    q /= q.sum()
    t = [threshold(zp, zq, y) for y in range(V)]
    law = np.zeros(V)
    for toks in itertools.product(range(V), repeat=m):
        w_tok = float(np.prod([q[y] for y in toks]))
        if w_tok == 0.0:
            continue
        for pattern in itertools.product((True, False), repeat=m):
            w = w_tok
            u = [0.5]
            for y, ok in zip(toks, pattern):
                w *= t[y] if ok else 1.0 - t[y]
                u.append(t[y] * 0.5 if ok else (1.0 + t[y]) * 0.5)
            if w == 0.0:
                continue
            r = run(zp, zq, toks, u, want_dist=True)
            if r["accept_len"][0] == 1:
                law[r["out_tokens"][0, 0]] += w
            else:
                assert r["accept_len"][0] == 0
                law += w * r["final_dist"][0]
    return law


def closed_form(p, q, m):
    a = np.minimum(p, q)
    beta = a.sum()
    rest = (1.0 - beta) ** m
    return a * (1.0 - rest) / beta + rest * p


def test_single_child_worked_case():
    """p = (0.5, 0.5), q = (0.9, 0.1), one child: 0.7 for token 0."""
    zp = f32(np.log([0.5, 0.5]))
    zq = f32(np.log([0.9, 0.1]))
    law = first_token_law(zp, zq, 1)
    p = np.exp(zp.astype(np.float64))
    p /= p.sum()
    q = np.exp(zq.astype(np.float64))
    q /= q.sum()
    assert np.allclose(law, closed_form(p, q, 1), atol=1e-12)
    assert abs(law[0] - 0.7) < 1e-6 and abs(law[1] - 0.3) < 1e-6


@pytest.mark.parametrize("m", [1, 2, 3])
@pytest.mark.parametrize("seed", range(3))
def test_enumerated_law_equals_closed_form(m, seed):
    rng = np.random.default_rng(900 + 10 * m + seed)
    V = 3 if m == 3 else 4
    zp = f32(rng.normal(0, 1.0, V))
    zq = f32(zp + rng.normal(0, 1.0, V))
    p = np.exp(zp.astype(np.float64) - zp.max())
    p /= p.sum()
    q = np.exp(zq.astype(np.float64) - zq.max())
    q /= q.sum()
    law = first_token_law(zp, zq, m)
    assert abs(law.sum() - 1.0) < 1e-12
    assert np.allclose(law, closed_form(p, q, m), atol=1e-12)
    # and it is not the target law: the rule is not lossless
    tv = 0.5 * np.abs(law - p).sum()
    assert tv > 1e-3, tv


def test_equal_distributions_give_the_target_law():
    """q = p: every child passes (beta = 1) and the law is p."""
    zp = f32([0.3, -1.0, 0.8])
    law = first_token_law(zp, zp.copy(), 2)
    p = np.exp(zp.astype(np.float64) - zp.max())
    p /= p.sum()
    assert np.allclose(law, p, atol=1e-12)
