"""CPU checks of the validity test that GPU tree construction uses for
near-tie requests (test_gpu_treebuild.check_best_first), and pins of the
oracle's tree scorer.  The oracle's own trees must pass; a tree with a
planted mistake must fail."""
import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
import synth
from test_gpu_treebuild import check_best_first


def _tree(seed, dtype="f32", W=3, N=3, budget=25):
    M = synth.complete_tree_rows(W, N)
    d = synth.treebuild_inputs(2, M, 200, dtype, T=0.9, logits=("gumbel", 2.0), seed=seed)
    o = oracle.tree_build(d["logits"], d["T"], W, N, budget, dtype=dtype)
    g = dict(parents=o["parents"].copy(), tokens=o["tokens"].copy(), rows=o["rows"].copy(),
             score=o["score"].copy(), n=o["n"].copy())
    return d, g, W, N, budget


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_trees_pass(seed, dtype):
    d, g, W, N, budget = _tree(300 + seed, dtype)
    for r in range(2):
        check_best_first(g, r, d, W, N, budget, None)


def test_tree_score_matches_scipy_along_paths():
    """Eq. 15 from an independent library: the sum of scipy log_softmax
    values along each node's path, each token in its parent's row."""
    d, g, W, N, budget = _tree(310)
    sc = oracle.tree_score(d["logits"], g["parents"], g["tokens"], g["rows"], g["n"], d["T"])
    lq = log_softmax(d["logits"].astype(np.float64) / d["T"], axis=2)
    for r in range(2):
        want = np.full(budget, -np.inf)
        want[0] = 0.0
        for j in range(1, int(g["n"][r])):
            p = g["parents"][r, j]
            want[j] = want[p] + lq[r, g["rows"][r, p], g["tokens"][r, j]]
        assert np.allclose(sc[r], want, rtol=0, atol=1e-12)
    bad = g["parents"].copy()
    bad[0, 3] = 5  # a parent after its child
    sc = oracle.tree_score(d["logits"], bad, g["tokens"], g["rows"], g["n"], d["T"])
    assert np.isnan(sc[0]).all() and np.isfinite(sc[1, 0])


def test_planted_mistakes_fail():
    d, g, W, N, budget = _tree(320)
    r = 0
    n = int(g["n"][r])
    # a child token that is not among the row's best
    bad = {k: v.copy() for k, v in g.items()}
    bad["tokens"][r, 2] = (bad["tokens"][r, 2] + 1) % 200
    while bad["tokens"][r, 2] in g["tokens"][r, 1:4]:
        bad["tokens"][r, 2] = (bad["tokens"][r, 2] + 1) % 200
    with pytest.raises(AssertionError):
        check_best_first(bad, r, d, W, N, budget, None)
    # a score that disagrees with the tree
    bad = {k: v.copy() for k, v in g.items()}
    bad["score"][r, n - 1] += 1e-3
    with pytest.raises(AssertionError):
        check_best_first(bad, r, d, W, N, budget, None)
    # the second expansion taken from the worst child of the root instead of
    # the best: rebuild by hand so the tree is otherwise well formed
    root_kids = [j for j in range(1, n) if g["parents"][r, j] == 0]
    worst = root_kids[-1]
    M = d["logits"].shape[1]
    z = d["logits"][r]
    cand = [int(t) for t in np.argsort(-z[g["rows"][r, worst]].astype(np.float64),
                                       kind="stable")[:W]]
    bad = {k: v.copy() for k, v in g.items()}
    e = 1 + len(root_kids)
    for c, t in enumerate(cand):
        bad["parents"][r, e + c] = worst
        bad["tokens"][r, e + c] = t
        ch = g["rows"][r, worst] * W + 1 + c
        bad["rows"][r, e + c] = ch if ch < M else -1
    bad["n"][r] = e + len(cand)
    bad["parents"][r, bad["n"][r]:] = -1
    bad["tokens"][r, bad["n"][r]:] = -1
    bad["rows"][r, bad["n"][r]:] = -1
    bad["score"][r] = oracle.tree_score(d["logits"][r:r + 1], bad["parents"][r:r + 1],
                                        bad["tokens"][r:r + 1], bad["rows"][r:r + 1],
                                        bad["n"][r:r + 1], d["T"])[0]
    assert np.isfinite(bad["score"][r, :bad["n"][r]]).all()
    with pytest.raises(AssertionError):
        check_best_first(bad, r, d, W, N, budget, None)
