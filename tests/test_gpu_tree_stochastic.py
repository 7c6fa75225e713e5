"""GPU parity of spec_verify_tree_stochastic against the fp64 oracle (needs an
MI355X).  accept_len, accept_node and out_tokens must be bit-exact except in
requests where one of the oracle's decisions lies within 1e-6 of its
threshold (a node test whose parent is accepted, or the draw): those are
counted and must give one of the outcomes the oracle produces with that
uniform moved just outside the band on either side.  final_dist agrees to
1e-5 absolute."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_stree, require_gpu, to_dev, to_dev_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_stree(d, want_dist=False, workspace=None):
    torch, sv = require_gpu()
    acc, node, out, dist = sv.spec_verify_tree_stochastic(
        to_dev_logits(d["target"], d["dtype"]), to_dev_logits(d["draft"], d["dtype"]),
        to_dev(d["parents"], np.int32), to_dev(d["tokens"], np.int32),
        to_dev(d["uniforms"], np.float32), d["T"], want_dist=want_dist, workspace=workspace)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), accept_node=node.cpu().numpy(),
                out_tokens=out.cpu().numpy(), final_dist=None if dist is None else dist.cpu().numpy())


def run_case(d, label, want_dist=True):
    B = d["target"].shape[0]
    print(f"[case] {label} B={B} n={d['target'].shape[1]} V={d['V']} {d['dtype']} T={d['T']}",
          flush=True)
    g = gpu_stree(d, want_dist=want_dist)
    o = oracle.tree_stochastic(d["target"], d["draft"], d["parents"], d["tokens"], d["uniforms"],
                               d["T"], dtype=d["dtype"], want_dist=want_dist)
    compare_stree(g, o, label, want_dist, d)
    return g, o


SHAPES = [(1, 1, 7), (2, 5, 1), (3, 2, 100), (5, 17, 1000), (2, 64, 5003), (4, 33, 151937), (2, 1024, 300),
          (16, 8, 4096)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}n{n}V{v}" for b, n, v in SHAPES])
def test_shapes(shape, dtype):
    B, n, V = shape
    d = synth.stree_inputs(B, n, V, dtype, T=0.9, noise=0.7, seed=6000 + B + n + V)
    run_case(d, f"st-{shape}-{dtype}")


@pytest.mark.parametrize("T", [0.05, 0.7, 5.0])
def test_temperatures(T):
    d = synth.stree_inputs(6, 40, 3000, "bf16", T=T, noise=0.5, seed=int(T * 100))
    run_case(d, f"st-T{T}")


def test_workload_full_size_sample():
    d = synth.stree_config_inputs(seed=9100, B=4)
    run_case(d, "st-workload-B4")


@pytest.mark.parametrize("seed", [9101, 9102, 9103])
def test_workload_bench_launch(seed):
    """The whole workload as bench.py times it (64 requests: the same chunk
    runs and grids, no final_dist), every request checked against the
    oracle."""
    d = synth.stree_config_inputs(seed=seed)
    print(f"[case] st-bench-launch seed {seed} B={d['target'].shape[0]}", flush=True)
    g = gpu_stree(d, want_dist=False)
    o = oracle.tree_stochastic(d["target"], d["draft"], d["parents"], d["tokens"],
                               d["uniforms"], d["T"], dtype=d["dtype"])
    compare_stree(g, o, f"st-bench-launch-s{seed}", False, d)


def test_one_hot_targets_equal_greedy_verification():
    """One-hot target rows make every test certain: the result must equal
    greedy tree verification of the same tree (on the GPU as well)."""
    torch, sv = require_gpu()
    B, n, V = 6, 50, 700
    d = synth.tree_inputs(B, n, V, seed=31)
    amax = np.argmax(synth.bf16_to_f32(d["target"]), axis=2)
    tgt = np.full((B, n, V), -np.inf, np.float32)
    np.put_along_axis(tgt, amax[..., None], 0.0, axis=2)
    rng = np.random.default_rng(32)
    e = dict(target=synth.bf16_bits(tgt), draft=synth.bf16_bits(rng.normal(0, 1, (B, n, V))),
             parents=d["parents"], tokens=d["tokens"],
             uniforms=rng.random((B, n)).astype(np.float32), V=V, dtype="bf16", T=1.0)
    g = gpu_stree(e)
    acc, node, out = sv.spec_verify_tree_greedy(to_dev_logits(e["target"], "bf16"),
                                                to_dev(e["parents"], np.int32),
                                                to_dev(e["tokens"], np.int32))
    torch.cuda.synchronize()
    assert np.array_equal(g["accept_len"], acc.cpu().numpy())
    assert np.array_equal(g["accept_node"], node.cpu().numpy())
    assert np.array_equal(g["out_tokens"], out.cpu().numpy())


def test_invalid_and_masked():
    rng = np.random.default_rng(33)
    B, n, V = 7, 9, 500
    d = synth.stree_inputs(B, n, V, "f32", T=1.0, seed=33)
    t, q, par, tok = d["target"], d["draft"], d["parents"], d["tokens"]
    par[1, 4] = 6           # a parent after its child
    tok[2, 3] = V           # a token out of range
    q[3, 2, 7] = np.nan     # a NaN draft logit
    t[4, 8, :] = -np.inf    # a target row without a finite logit
    t[5, par[5, 3], tok[5, 3]] = -np.inf  # a token the target rules out: always rejected
    q[6, par[6, 2], tok[6, 2]] = -np.inf  # a token the draft rules out: always accepted
    run_case(d, "st-invalid-masked")
