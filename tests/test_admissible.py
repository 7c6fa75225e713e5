"""The band-validity search (tests/admissible.py) on the CPU: with a uniform
placed exactly on a decision boundary, the admissible outcomes are the two
the oracle gives on either side of it, and nothing else is accepted."""
import numpy as np

import admissible
import oracle
import synth


def test_test_on_boundary_admits_both_decisions():
    for seed in range(5, 50):
        d = synth.chain_inputs(1, 3, 40, "f32", T=1.0, seed=seed)
        r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], 1.0)
        if 0.05 < r["ratios"][0, 1] < 0.95:
            break
    u = np.array([0.0, 0.0, 0.0, 0.37])
    u[1] = r["ratios"][0, 1]  # on test 1's threshold: u = r rejects, just below accepts
    leaves = admissible.chain_leaves(d["target"][0], d["draft"][0], d["draft_tokens"][0], u, 1.0,
                                     "f32")
    ks = sorted({leaf[1] for leaf in leaves})
    assert 1 in ks and any(k >= 2 for k in ks)
    for leaf in leaves:
        if leaf[0] == "exact":
            assert admissible.matches(leaves, leaf[1], leaf[2])
    # an outcome that no side of the boundary gives is refused
    assert not admissible.matches(leaves, 0, (int(d["draft_tokens"][0, 0]) + 1,) + (-1,) * 3)


def test_draw_on_a_breakpoint_admits_the_neighbouring_tokens():
    d = synth.chain_inputs(1, 2, 30, "f32", T=1.0, seed=6)
    u = np.array([0.0, 0.0, 0.5])  # both tests pass: the draw is from the bonus row
    r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], u[None], 1.0, want_dist=True)
    assert r["accept_len"][0] == 2
    C = np.cumsum(r["final_dist"][0])
    u[2] = C[10]  # exactly on the breakpoint between tokens 10 and 11
    leaves = admissible.chain_leaves(d["target"][0], d["draft"][0], d["draft_tokens"][0], u, 1.0,
                                     "f32")
    assert [leaf[0] for leaf in leaves] == ["range"]
    prefix = tuple(int(x) for x in d["draft_tokens"][0])
    assert admissible.matches(leaves, 2, prefix + (10,))
    assert admissible.matches(leaves, 2, prefix + (11,))
    assert not admissible.matches(leaves, 2, prefix + (12,))
    assert not admissible.matches(leaves, 1, prefix[:1] + (10, -1))


def test_stochastic_tree_node_on_boundary():
    for seed in range(7, 60):
        d = synth.stree_inputs(1, 6, 25, "f32", T=1.0, noise=0.5, seed=seed)
        o = oracle.tree_stochastic(d["target"], d["draft"], d["parents"], d["tokens"],
                                   np.zeros((1, 6), np.float32), 1.0, dtype="f32")
        j = 1  # a child of the root: its parent is always accepted
        if 0.05 < o["alpha"][0, j] < 0.95:
            break
    u = np.zeros(6)
    u[0] = 0.4
    u[j] = o["alpha"][0, j]
    leaves = admissible.stree_leaves(d["target"][0], d["draft"][0], d["parents"][0],
                                     d["tokens"][0], u, 1.0, "f32")
    assert len(leaves) >= 2
    for leaf in leaves:
        if leaf[0] == "exact":
            assert admissible.matches(leaves, leaf[1], leaf[2])
