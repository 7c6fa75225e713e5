"""GPU parity of spec_verify_tree_greedy against the oracle (needs an MI355X).
Tree results have no tolerance: accept lengths, nodes and tokens must match
exactly."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_tree, gpu_tree, require_gpu

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_case(d, label, dtype="bf16"):
    print(f"[case] {label} B={d['B']} n={d['n']} V={d['V']} {dtype}", flush=True)
    d = dict(d, dtype=dtype)
    g = gpu_tree(d)
    o = oracle.tree_greedy(d["target"], d["parents"], d["tokens"], dtype=dtype)
    compare_tree(g, o, label)
    return g, o


@pytest.mark.parametrize("seeds", [range(i, i + 5) for i in range(0, 20, 5)],
                         ids=[f"s{i}-{i + 4}" for i in range(0, 20, 5)])
def test_config4_full_size(seeds):
    """20 seeded rounds of the 64 x 64-node workload, bit-exact."""
    for s in seeds:
        d = synth.config_inputs(4, seed=4000 + s)
        g, _ = run_case(d, f"config4-s{s}")
        assert (g["accept_len"] >= 0).all()


TREE_SHAPES = [(4, 1, 100), (8, 2, 7), (6, 17, 1000), (3, 64, 151937), (2, 1024, 300),
               (5, 100, 4097)]


@pytest.mark.parametrize("shape", TREE_SHAPES, ids=[f"B{b}n{n}V{v}" for b, n, v in TREE_SHAPES])
def test_shapes(shape):
    B, n, V = shape
    d = synth.tree_inputs(B, n, V, max_depth=min(16, n), max_children=4, seed=41)
    run_case(d, f"tree{shape}")


def test_f32_rows():
    d = synth.tree_inputs(6, 40, 3001, seed=42)
    z = synth.bf16_to_f32(d["target"]).copy()
    z += np.random.default_rng(42).normal(0, 1e-3, z.shape).astype(np.float32)
    d["target"] = z
    run_case(d, "tree-f32", dtype="f32")


def test_ties_and_duplicates():
    rng = np.random.default_rng(43)
    B, n, V = 500, 12, 9
    par = np.full((B, n), -1, np.int32)
    for j in range(1, n):
        par[:, j] = rng.integers(0, j, B)
    z = rng.integers(-3, 3, (B, n, V)).astype(np.float32)
    amax = np.argmax(z, axis=2)
    tok = np.where(rng.random((B, n)) < 0.7, np.take_along_axis(amax, par.clip(0), 1),
                   rng.integers(0, V, (B, n))).astype(np.int32)
    d = dict(target=synth.bf16_bits(z), parents=par, tokens=tok, B=B, n=n, V=V)
    run_case(d, "ties")


def test_path_shaped():
    rng = np.random.default_rng(44)
    B, n, V = 64, 33, 5000
    d = synth.tree_inputs(B, n, V, max_depth=32, max_children=1, seed=44)
    assert (d["parents"][:, 1:] == np.arange(n - 1)).all()
    run_case(d, "path")


def test_fig5():
    g = json.load(open(os.path.join(GOLD, "fig5_tree.json")))
    vocab = {w: i for i, w in enumerate(g["vocab"])}
    V = len(vocab)
    par = np.array([nd["parent"] for nd in g["nodes"]], np.int32)
    tok = np.array([vocab[nd["token"]] for nd in g["nodes"]], np.int32)
    amax = np.array([vocab[nd["target_argmax"]] for nd in g["nodes"]])
    z = np.random.default_rng(0).normal(0, 1, (len(par), V)).astype(np.float32)
    z[np.arange(len(par)), amax] = 10.0
    d = dict(target=synth.bf16_bits(z)[None], parents=par[None], tokens=tok[None], B=1,
             n=len(par), V=V)
    res, _ = run_case(d, "fig5")
    assert res["accept_len"][0] == g["expected_accept_len"]


@pytest.mark.parametrize("kind", ["root_parent", "forward_parent", "token_range", "nan",
                                  "posinf", "allneginf"])
def test_invalid_requests(kind):
    d = synth.tree_inputs(3, 10, 4000, seed=45)
    if kind == "root_parent":
        d["parents"][1, 0] = 0
    elif kind == "forward_parent":
        d["parents"][1, 4] = 7
    elif kind == "token_range":
        d["tokens"][1, 5] = 4000
    elif kind == "nan":
        d["target"][1, 6, 3] = 0x7FC0
    elif kind == "posinf":
        d["target"][1, 2, 3999] = 0x7F80
    else:
        d["target"][1, 3, :] = 0xFF80
    g, _ = run_case(d, f"invalid-{kind}")
    assert g["accept_len"][1] == -1 and (g["out_tokens"][1] == -1).all()


def test_repeated_calls():
    torch, sv = require_gpu()
    d = synth.tree_inputs(16, 64, 20000, seed=46)
    ws = torch.full((sv.spec_verify_tree_greedy_workspace_bytes(16, 64, 20000, 1),), 0xA5,
                    dtype=torch.uint8, device="cuda")
    first = gpu_tree(dict(d, dtype="bf16"), workspace=ws)
    compare_tree(first, oracle.tree_greedy(d["target"], d["parents"], d["tokens"]), "reuse")
    for fill in (0x00, 0xFF):
        ws.fill_(fill)
        again = gpu_tree(dict(d, dtype="bf16"), workspace=ws)
        for k in first:
            assert np.array_equal(first[k], again[k])
