"""Pins of the oracle's greedy tree verification.  CPU only.

The rule ("JetSpec reading notes", tree verification, Fig. 5 and the greedy
note): at T = 0 a node is accepted iff its token equals the target argmax
after its parent's path and its parent is accepted; the deepest accepted node
wins; the target argmax after that node is the extra (bonus) token.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


def rows_with_argmax(amax, V, rng, ties=False):
    """bf16 rows whose lowest-index argmax is amax[j] (values drawn here)."""
    n = len(amax)
    z = rng.normal(0, 1, (n, V)).astype(np.float32)
    z[np.arange(n), amax] = 10.0
    if ties:
        for j in range(n):
            if amax[j] + 1 < V:
                z[j, amax[j] + 1:] = np.minimum(z[j, amax[j] + 1:], 10.0)
                z[j, V - 1] = 10.0 if amax[j] < V - 1 else z[j, V - 1]
    return bf16(z)


def brute_force(parents, tokens, amax):
    """For every node walk to the root checking each edge; keep the deepest
    fully matching node (lowest index on equal depth)."""
    n = len(parents)
    best, best_depth = 0, 0
    for j in range(1, n):
        ok, depth, v = True, 0, j
        while v != 0:
            p = parents[v]
            ok = ok and tokens[v] == amax[p]
            depth += 1
            v = p
        if ok and depth > best_depth:
            best, best_depth = j, depth
    path = []
    v = best
    while v != 0:
        path.append(int(tokens[v]))
        v = parents[v]
    return best, best_depth, path[::-1] + [int(amax[best])]


def test_fig5_example():
    g = json.load(open(os.path.join(GOLD, "fig5_tree.json")))
    vocab = {w: i for i, w in enumerate(g["vocab"])}
    V = len(vocab)
    nodes = g["nodes"]
    par = np.array([nd["parent"] for nd in nodes], np.int32)
    tok = np.array([vocab[nd["token"]] for nd in nodes], np.int32)
    amax = np.array([vocab[nd["target_argmax"]] for nd in nodes])
    rows = rows_with_argmax(amax, V, np.random.default_rng(0))
    r = oracle.tree_greedy(rows[None], par[None], tok[None])
    k = int(r["accept_len"][0])
    assert k == g["expected_accept_len"]
    out = [g["vocab"][t] for t in r["out_tokens"][0, :k + 1]]
    assert out == g["expected_path"] + [g["expected_bonus"]]
    assert k + 1 == g["expected_committed"]
    assert (r["amax"][0] == amax).all()


def test_random_trees_match_brute_force():
    """10^4 random small trees, with duplicate sibling tokens and tied maxima."""
    rng = np.random.default_rng(1)
    B, n, V = 10_000, 12, 5
    par = np.full((B, n), -1, np.int32)
    for j in range(1, n):
        par[:, j] = rng.integers(0, j, B)
    z = rng.integers(-3, 3, (B, n, V)).astype(np.float32)  # many ties
    amax_ref = np.argmax(z, axis=2)  # numpy: first occurrence on ties
    tok = np.where(rng.random((B, n)) < 0.7,
                   np.take_along_axis(amax_ref, par.clip(0), 1),
                   rng.integers(0, V, (B, n))).astype(np.int32)
    r = oracle.tree_greedy(bf16(z), par, tok)
    assert (r["amax"] == amax_ref).all()
    for b in range(B):
        node, depth, path = brute_force(par[b], tok[b], amax_ref[b])
        assert r["accept_node"][b] == node
        assert r["accept_len"][b] == depth
        assert list(r["out_tokens"][b, :depth + 1]) == path
        assert (r["out_tokens"][b, depth + 1:] == -1).all()


def test_path_shaped_tree_is_chain_first_mismatch():
    """On a path the rule is the chain greedy rule: accept up to the first
    position whose token differs from the target argmax (the first-mismatch
    rule anchor replacement uses in JetSpec++)."""
    rng = np.random.default_rng(2)
    B, n, V = 500, 9, 7
    par = np.tile(np.arange(-1, n - 1, dtype=np.int32), (B, 1))
    z = rng.normal(0, 1, (B, n, V)).astype(np.float32)
    amax = np.argmax(synth.bf16_to_f32(bf16(z)), axis=2)
    tok = np.zeros((B, n), np.int32)
    tok[:, 1:] = np.where(rng.random((B, n - 1)) < 0.8, amax[:, :-1],
                          rng.integers(0, V, (B, n - 1)))
    r = oracle.tree_greedy(bf16(z), par, tok)
    for b in range(B):
        k = 0
        while k + 1 < n and tok[b, k + 1] == amax[b, k]:
            k += 1
        assert r["accept_len"][b] == k
        assert r["out_tokens"][b, k] == amax[b, k]


def test_root_only_tree():
    rng = np.random.default_rng(3)
    z = bf16(rng.normal(0, 1, (4, 1, 50)))
    r = oracle.tree_greedy(z, np.full((4, 1), -1, np.int32), np.zeros((4, 1), np.int32))
    assert (r["accept_len"] == 0).all() and (r["accept_node"] == 0).all()
    assert (r["out_tokens"][:, 0] == np.argmax(synth.bf16_to_f32(z)[:, 0], axis=1)).all()


def test_tie_goes_to_lowest_token_and_node():
    V = 6
    z = np.zeros((3, V), np.float32)
    z[0, [2, 4]] = 5.0  # tied maximum at 2 and 4 -> argmax 2
    z[1, 1] = 3.0
    z[2, 3] = 3.0
    par = np.array([-1, 0, 0], np.int32)
    tok = np.array([0, 2, 2], np.int32)  # duplicate siblings, both accepted
    r = oracle.tree_greedy(bf16(z)[None], par[None], tok[None])
    assert r["amax"][0, 0] == 2
    assert r["accept_node"][0] == 1 and r["accept_len"][0] == 1
    assert list(r["out_tokens"][0]) == [2, 1, -1]
    tok = np.array([0, 4, 4], np.int32)  # the later of two tied maxima is rejected
    r = oracle.tree_greedy(bf16(z)[None], par[None], tok[None])
    assert r["accept_len"][0] == 0 and list(r["out_tokens"][0]) == [2, -1, -1]


def test_negative_infinity_allowed_and_all_masked_invalid():
    V = 5
    z = np.full((2, V), -np.inf, np.float32)
    z[0, 3] = -100.0
    z[1, 0] = 1.0
    par = np.array([-1, 0], np.int32)
    tok = np.array([0, 3], np.int32)
    r = oracle.tree_greedy(bf16(z)[None], par[None], tok[None])
    assert r["accept_len"][0] == 1 and list(r["out_tokens"][0]) == [3, 0]
    z[1, 0] = -np.inf
    r = oracle.tree_greedy(bf16(z)[None], par[None], tok[None])
    assert r["accept_len"][0] == -1 and (r["out_tokens"][0] == -1).all()


@pytest.mark.parametrize("kind", ["root_parent", "forward_parent", "self_parent",
                                  "token_range", "nan", "posinf"])
def test_invalid_request_flagged_alone(kind):
    d = synth.tree_inputs(B=3, n=10, V=40, seed=4)
    tgt, par, tok = d["target"].copy(), d["parents"].copy(), d["tokens"].copy()
    if kind == "root_parent":
        par[1, 0] = 0
    elif kind == "forward_parent":
        par[1, 4] = 7
    elif kind == "self_parent":
        par[1, 4] = 4
    elif kind == "token_range":
        tok[1, 5] = 40
    elif kind == "nan":
        tgt[1, 6, 3] = 0x7FC0
    else:
        tgt[1, 2, 9] = 0x7F80
    ref = oracle.tree_greedy(d["target"], d["parents"], d["tokens"])
    r = oracle.tree_greedy(tgt, par, tok)
    assert r["accept_len"][1] == -1 and (r["out_tokens"][1] == -1).all()
    for b in (0, 2):
        assert r["accept_len"][b] == ref["accept_len"][b]
        assert (r["out_tokens"][b] == ref["out_tokens"][b]).all()


def test_anchor_token_is_not_checked():
    d = synth.tree_inputs(B=2, n=8, V=30, seed=5)
    tok = d["tokens"].copy()
    tok[:, 0] = 12345  # out of range, but node 0's token is the anchor
    a = oracle.tree_greedy(d["target"], d["parents"], d["tokens"])
    b = oracle.tree_greedy(d["target"], d["parents"], tok)
    assert (a["accept_len"] == b["accept_len"]).all() and (a["accept_len"] >= 0).all()
