"""Outcomes a correct implementation may return for a block whose decisions
lie within BAND of their boundaries.

A decision whose uniform is within BAND of its threshold (a ratio test, a
point-mass test, a tree-node test) or of a CDF breakpoint (the final draw)
can go either way under rounding of order 1e-7.  For such a block the oracle
is run again with that uniform moved 2*BAND to each side of the boundary,
every other uniform unchanged, and this repeats on each resulting path until
no decision on it is inside the band.  The admissible outcomes are the leaves
of that search; an implementation's result must be one of them:

  ("exact", k, tokens)         the whole output must be equal;
  ("range", k, prefix, lo, hi) a banded final draw: the tokens before the
                               draw must be equal, and the drawn token must
                               lie in [lo, hi] with positive probability under
                               the draw's distribution (the tokens of u moved
                               2*BAND down and up bound every token whose CDF
                               interval meets the band);
  ("any", k, prefix)           a rejection whose residual mass is zero in the
                               oracle's arithmetic (possible only at a test
                               within rounding of r = 1): the drawn token is
                               not determined by the rule, only the prefix.

Only the oracle computes outcomes here; this module decides where to move
the uniforms, from the oracle's own reported test probabilities.
"""
from __future__ import annotations

import numpy as np

BAND = 1e-6
_TOP = float(np.nextafter(1.0, 0.0))


def _sides(u, r):
    """Uniform values just below (accept) and at or above (reject) a test
    threshold r; None where that side cannot occur for u in [0, 1)."""
    acc = max(0.0, r - 2 * BAND) if r > 0.0 else None
    if r >= 1.0:
        rej = None
    else:
        rej = r + 2 * BAND if r + 2 * BAND < 1.0 else r
    return acc, rej


def _draw_sides(u):
    return max(0.0, u - 2 * BAND), min(_TOP, u + 2 * BAND)


def _search(run, u, tests, leaves, forced=frozenset()):
    """run(u float64 vector, want_dist=False) -> oracle dict for one block
    (B = 1), with draw_pos (position of the drawn token in out_tokens),
    draw_index (index of the draw's uniform) and fallback added;
    tests(res) -> list of (index into u, threshold) of the decisions the
    result depends on, in decision order.  `forced` holds the indices of
    uniforms already moved to one side of their boundary (not branched on
    again, even where the moved value is still within BAND because the
    boundary is within 2*BAND of 0 or 1)."""
    res = run(u)
    k = int(res["accept_len"][0])
    out = res["out_tokens"][0]
    if k < 0:
        leaves.append(("exact", k, tuple(out.tolist())))
        return
    for idx, r in tests(res, u):
        if idx not in forced and abs(u[idx] - r) < BAND:
            acc, rej = _sides(u[idx], r)
            for side in (acc, rej):
                if side is None:
                    continue
                v = u.copy()
                v[idx] = side
                _search(run, v, tests, leaves, forced | {idx})
            return
    prefix = tuple(out[:res["draw_pos"]].tolist())
    if res["fallback"]:
        leaves.append(("any", k, prefix))
        return
    if res["margin"][0] < BAND:
        di = res["draw_index"]
        lo_u, hi_u = _draw_sides(u[di])
        toks = []
        for side in (lo_u, hi_u):
            v = u.copy()
            v[di] = side
            rr = run(v)
            assert int(rr["accept_len"][0]) == k, "moving the draw's uniform changed a test"
            toks.append(int(rr["out_tokens"][0][res["draw_pos"]]))
        leaves.append(("range", k, prefix, min(toks), max(toks), u.copy(), run))
        return
    leaves.append(("exact", k, tuple(out.tolist())))


def matches(leaves, k, out):
    """Whether (k, out) is one of the admissible outcomes.  A drawn token
    strictly inside a range, which the oracle has not produced itself, must
    have positive probability in the oracle's draw distribution on that
    path."""
    out = tuple(int(x) for x in out)
    for leaf in leaves:
        kind = leaf[0]
        if leaf[1] != k:
            continue
        if kind == "exact":
            if out == leaf[2]:
                return True
            continue
        prefix = leaf[2]
        n = len(prefix)
        if out[:n] != prefix:
            continue
        if kind == "any":
            return True
        lo, hi, u, run = leaf[3], leaf[4], leaf[5], leaf[6]
        t = out[n]
        if t in (lo, hi):
            return True
        if lo < t < hi and run(u, want_dist=True)["final_dist"][0][t] > 0.0:
            return True
    return False


def describe(leaves):
    return [leaf[:5] for leaf in leaves]


# ------------------------------------------------------------------ chains --

def chain_leaves(target, draft, tokens, uniforms, T, dtype, pointmass=False):
    """Admissible outcomes of one chain block (target [g+1, V], draft [g, V]
    or None for point mass, tokens [g], uniforms [g+1])."""
    import oracle

    g = tokens.shape[0]
    tgt, tok = target[None], tokens[None]
    drf = None if pointmass else draft[None]

    def run(u, want_dist=False):
        if pointmass:
            res = oracle.chain_pointmass(tgt, tok, u[None], T, dtype=dtype, want_dist=want_dist,
                                         threads=1)
        else:
            res = oracle.chain(tgt, drf, tok, u[None], T, dtype=dtype, want_dist=want_dist,
                               threads=1)
        k = int(res["accept_len"][0])
        res["draw_pos"] = max(k, 0)
        res["draw_index"] = g
        res["fallback"] = bool(res["fallback"][0])
        return res

    def tests(res, u):
        k = int(res["accept_len"][0])
        last = min(k, g - 1)
        return [(i, float(res["ratios"][0][i])) for i in range(last + 1)]

    leaves = []
    _search(run, np.asarray(uniforms, np.float64).copy(), tests, leaves)
    return leaves


# ------------------------------------------------------ stochastic trees --

def stree_leaves(target, draft, parents, tokens, uniforms, T, dtype):
    """Admissible outcomes of one stochastic-tree request (target, draft
    [n, V], parents, tokens, uniforms [n]).  The tests branched on are those
    of nodes whose parent counts as accepted (a node's test decides nothing
    when its parent is rejected)."""
    import oracle

    n = parents.shape[0]

    def run(u, want_dist=False):
        res = oracle.tree_stochastic(target[None], draft[None], parents[None], tokens[None],
                                     u[None], T, dtype=dtype, want_dist=want_dist)
        res["draw_pos"] = max(int(res["accept_len"][0]), 0)
        res["draw_index"] = 0
        res["fallback"] = False
        return res

    def tests(res, u):
        a = res["alpha"][0]
        acc = np.zeros(n, bool)
        acc[0] = True
        live = []
        for j in range(1, n):
            p = parents[j]
            if acc[p]:
                live.append((j, float(a[j])))
            acc[j] = acc[p] and u[j] < a[j]
        return live

    leaves = []
    _search(run, np.asarray(uniforms, np.float64).copy(), tests, leaves)
    return leaves
