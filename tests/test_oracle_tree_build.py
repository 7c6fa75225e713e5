"""Pins of the oracle's draft-tree construction against what the pages and the
mathematics fix.  CPU only.

"JetSpec" reading notes, Algorithm 1 (best-first tree construction under a
node budget, top-W children per node, nodes at depth N are leaves) with the
branch score of Eq. 15 (the sum of draft log probabilities along the path).
The oracle is a priority-queue search; the brute force below takes another
route: every log probability is <= 0, so scores fall along every path and the
best-first order is the order of all expandable potential nodes by
descending score.  Expanding them in that order until the budget is spent
must give the oracle's tree exactly (on inputs without score ties).
"""
import numpy as np
import pytest
from scipy.special import log_softmax

import oracle


def f32(x):
    return np.asarray(x, dtype=np.float32)


def child_of(m, j, W, M, child_row):
    if child_row is not None:
        return int(child_row[m, j])
    c = m * W + 1 + j
    return c if c < M else -1


def brute_tree(z, T, W, N, budget, child_row=None):
    """Best-first tree by sorting the potential tree (see the module note)."""
    M, V = z.shape
    lq = log_softmax(z.astype(np.float64) / T, axis=1)
    top = []
    for m in range(M):
        order = sorted((v for v in range(V) if np.isfinite(z[m, v])), key=lambda v: (-z[m, v], v))
        top.append(order[:W])
    # the potential tree: (path, row, depth, score); children in rank order
    nodes = [((), 0, 0, 0.0)]
    frontier = [0]
    while frontier:
        nxt = []
        for i in frontier:
            path, row, depth, s = nodes[i]
            if depth >= N or row < 0:
                continue
            for j, y in enumerate(top[row]):
                nodes.append((path + (y,), child_of(row, j, W, M, child_row), depth + 1, s + lq[row, y]))
                nxt.append(len(nodes) - 1)
        frontier = nxt
    expandable = [i for i, (_, row, depth, _) in enumerate(nodes) if depth < N and row >= 0]
    expandable.sort(key=lambda i: -nodes[i][3])
    ids = {(): 0}
    par, tok, rows, sc = [-1], [-1], [0], [0.0]
    for i in expandable:
        if len(par) >= budget:
            break
        path, row, depth, s = nodes[i]
        assert path in ids  # its parent scored higher, so it was expanded first
        for j, y in enumerate(top[row]):
            if len(par) >= budget:
                break
            ids[path + (y,)] = len(par)
            par.append(ids[path])
            tok.append(y)
            rows.append(child_of(row, j, W, M, child_row))
            sc.append(s + lq[row, y])
    return np.array(par), np.array(tok), np.array(rows), np.array(sc)


def check_against_brute(z, T, W, N, budget, child_row=None):
    r = oracle.tree_build(z[None], T, W, N, budget, child_row=child_row)
    n = int(r["n"][0])
    par, tok, rows, sc = brute_tree(z, T, W, N, budget, child_row)
    assert n == len(par)
    assert r["parents"][0, :n].tolist() == par.tolist()
    assert r["tokens"][0, :n].tolist() == tok.tolist()
    assert r["rows"][0, :n].tolist() == rows.tolist()
    assert np.abs(r["score"][0, :n] - sc).max() < 1e-12
    assert (r["parents"][0, n:] == -1).all() and (r["score"][0, n:] == -np.inf).all()
    return r


@pytest.mark.parametrize("seed", range(12))
def test_equals_sorted_expansion_of_the_potential_tree(seed):
    rng = np.random.default_rng(600 + seed)
    W = int(rng.integers(1, 5))
    N = int(rng.integers(1, 5))
    M = sum(W ** d for d in range(N))  # every node above depth N has a row
    V = int(rng.integers(W, 60))
    z = f32(rng.normal(0, 2.0, (M, V)))
    budget = int(rng.integers(1, sum(W ** d for d in range(N + 1)) + 3))
    check_against_brute(z, float(rng.choice([0.5, 1.0, 2.0])), W, N, budget)


@pytest.mark.parametrize("seed", range(6))
def test_sparse_child_map(seed):
    """An explicit map in which only some children have rows: the others are
    added but never expanded, and rows may be shared or out of BFS order."""
    rng = np.random.default_rng(700 + seed)
    W, N, M, V = 3, 4, 12, 40
    z = f32(rng.normal(0, 1.5, (M, V)))
    cr = rng.integers(1, M, (M, W)).astype(np.int32)
    cr[rng.random((M, W)) < 0.4] = -1
    check_against_brute(z, 1.0, W, N, int(rng.integers(2, 30)), child_row=cr)


def test_implicit_map_equals_explicit_bfs_map():
    rng = np.random.default_rng(11)
    W, N, V = 3, 3, 30
    M = 1 + 3 + 9
    z = f32(rng.normal(0, 1, (M, V)))
    cr = np.array([[m * W + 1 + j if m * W + 1 + j < M else -1 for j in range(W)] for m in range(M)],
                  np.int32)
    a = oracle.tree_build(z[None], 1.0, W, N, 20)
    b = oracle.tree_build(z[None], 1.0, W, N, 20, child_row=cr)
    for key in ("parents", "tokens", "rows", "score", "n"):
        assert np.array_equal(a[key], b[key])


def test_worked_example():
    """A hand-worked case.  V = 5, W = 2, N = 2, T = 1, rows for the root and
    its two children (M = 3):
      root  p = (.10, .50, .05, .30, .05): children token 1 (node 1, ln .5)
            and token 3 (node 2, ln .3);
      row 1 p = (.60, .05, .05, .20, .10): node 1 is expanded first (ln .5 is
            the best score): token 0 (node 3, ln .30) and token 3 (node 4, ln .10);
      row 2 p = (.10, .10, .70, .05, .05): node 2 is next (nodes 3 and 4 sit at
            depth N and are never expanded): token 2 (node 5, ln .21), then
            the tie at .10 goes to token 0 (node 6, ln .03).
    A budget of 6 stops after node 5; a budget of 8 leaves the full tree of
    7 nodes; N = 1 keeps the root's children only."""
    p = np.array([[.10, .50, .05, .30, .05], [.60, .05, .05, .20, .10], [.10, .10, .70, .05, .05]])
    z = f32(np.log(p))
    r = oracle.tree_build(z[None], 1.0, 2, 2, 6)
    assert r["n"][0] == 6
    assert r["parents"][0].tolist() == [-1, 0, 0, 1, 1, 2]
    assert r["tokens"][0].tolist() == [-1, 1, 3, 0, 3, 2]
    assert r["rows"][0].tolist() == [0, 1, 2, -1, -1, -1]
    want = np.log([1.0, .5, .3, .3, .1, .21])
    assert np.abs(r["score"][0] - want).max() < 1e-6
    r = oracle.tree_build(z[None], 1.0, 2, 2, 8)
    assert r["n"][0] == 7 and r["tokens"][0, 6] == 0 and r["parents"][0, 6] == 2
    assert abs(r["score"][0, 6] - np.log(.03)) < 1e-6
    r = oracle.tree_build(z[None], 1.0, 2, 1, 8)
    assert r["n"][0] == 3 and r["tokens"][0, :3].tolist() == [-1, 1, 3]


def test_width_one_is_the_greedy_chain():
    """W = 1: the tree is a path whose tokens are the argmax of rows 0, 1, ...
    (child 0 of row m is row m + 1), of length min(budget - 1, N)."""
    rng = np.random.default_rng(3)
    M, V = 6, 100
    z = f32(rng.normal(0, 1, (M, V)))
    for N, budget in [(6, 100), (6, 4), (3, 100)]:
        r = oracle.tree_build(z[None], 0.7, 1, N, budget)
        n = int(r["n"][0])
        assert n == min(budget, N + 1)
        assert r["parents"][0, :n].tolist() == [-1] + list(range(n - 1))
        assert r["tokens"][0, 1:n].tolist() == np.argmax(z[:n - 1], axis=1).tolist()


def test_budget_beyond_the_full_tree():
    """A budget above 1 + W + ... + W^N builds the complete tree: every node
    above depth N has exactly its W most probable tokens as children."""
    rng = np.random.default_rng(4)
    W, N, V = 3, 3, 25
    M = 1 + 3 + 9
    z = f32(rng.normal(0, 1, (M, V)))
    r = oracle.tree_build(z[None], 1.0, W, N, 100)
    n = int(r["n"][0])
    assert n == 1 + 3 + 9 + 27
    par, tok, rows = r["parents"][0, :n], r["tokens"][0, :n], r["rows"][0, :n]
    for v in range(n):
        kids = np.nonzero(par == v)[0]
        if rows[v] >= 0:
            want = np.argsort(-z[rows[v]], kind="stable")[:W]
            assert tok[kids].tolist() == want.tolist()
        else:
            assert len(kids) == 0


def test_masked_tokens_and_invalid_rows():
    """Tokens of probability 0 are not candidates (a row with one finite logit
    gives one child, of log probability 0); a row without a finite logit or
    with a NaN makes the request invalid."""
    V = 8
    z = np.full((3, V), -np.inf, np.float32)
    z[0, [2, 5]] = [1.0, 0.0]
    z[1, 4] = 3.0
    z[2, :] = 0.0
    r = oracle.tree_build(z[None], 1.0, 4, 2, 50)
    assert r["n"][0] == 1 + 2 + 1 + 4
    assert r["tokens"][0, 1:3].tolist() == [2, 5]
    assert r["tokens"][0, 3] == 4 and r["parents"][0, 3] == 1 and r["score"][0, 3] == r["score"][0, 1]
    bad = z.copy()
    bad[2, 3] = np.nan
    zz = np.stack([z, bad, np.full((3, V), -np.inf, np.float32)])
    r = oracle.tree_build(zz, 1.0, 4, 2, 50)
    assert r["n"].tolist() == [8, -1, -1]
    assert (r["parents"][1:] == -1).all() and (r["tokens"][1:] == -1).all()


def test_parent_arrays_suit_tree_verification():
    """parents[0] = -1 and 0 <= parents[j] < j, the layout greedy tree
    verification takes; depths never exceed N."""
    rng = np.random.default_rng(5)
    W, N, V = 4, 4, 64
    M = sum(W ** d for d in range(N))
    z = f32(rng.normal(0, 3, (5, M, V)))
    r = oracle.tree_build(z, 1.0, W, N, 40)
    for b in range(5):
        n = int(r["n"][b])
        par = r["parents"][b, :n]
        assert par[0] == -1 and all(0 <= par[j] < j for j in range(1, n))
        depth = np.zeros(n, int)
        for j in range(1, n):
            depth[j] = depth[par[j]] + 1
        assert depth.max() <= N
