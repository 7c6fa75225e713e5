"""One scratch workspace shared by calls of different sizes and entry points.

The library needs no initialised workspace: each call writes every workspace
byte it later reads.  Regression test for a workspace reused across shapes
and entry points and refilled with garbage bytes before each call: results
must match the oracle after every call."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_chain, compare_tree, gpu_chain, gpu_tree, require_gpu

pytestmark = pytest.mark.gpu


def test_workspace_reused_across_shapes_and_entry_points():
    torch, sv = require_gpu()
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    calls = [
        ("chain", synth.chain_inputs(3, 1, 1, "f32", seed=1)),
        ("tree", synth.tree_inputs(4, 64, 5003, seed=2)),
        ("chain", synth.chain_inputs(9, 7, 20000, "bf16", T=0.7, seed=3)),
        ("chain", synth.chain_inputs(2, 3, 5003, "f32", seed=4)),
        ("tree", synth.tree_inputs(2, 1024, 300, seed=5)),
        ("chain", synth.chain_inputs(16, 16, 4096, "bf16", T=1.2, seed=6)),
        ("tree", synth.tree_inputs(8, 17, 1000, seed=7)),
    ]
    fills = [0x00, 0xFF, 0xA5, 0x7F]
    for i, (kind, d) in enumerate(calls):
        print(f"[case] shared workspace call {i}: {kind}", flush=True)
        if kind == "chain":
            for want_dist in (False, True):
                ws.fill_(fills[(2 * i + int(want_dist)) % len(fills)])
                g = gpu_chain(d, want_dist=want_dist, workspace=ws)
                o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                                 dtype=d["dtype"], want_dist=want_dist)
                compare_chain(g, o, f"call{i}-dist{want_dist}", d=d)
        else:
            ws.fill_(fills[i % len(fills)])
            g = gpu_tree(dict(d, dtype="bf16"), workspace=ws)
            o = oracle.tree_greedy(d["target"], d["parents"], d["tokens"])
            compare_tree(g, o, f"call{i}")


def test_workspace_garbage_for_outcomes_and_tree_construction():
    """The same contract for spec_outcome_topk, spec_verify_chain_pointmass and
    spec_tree_build: a shared workspace refilled with garbage before every
    call, shapes changing between calls."""
    torch, sv = require_gpu()
    from gpu_util import (compare_outcomes, gpu_outcome, gpu_pointmass, to_dev,
                          to_dev_logits)
    from test_gpu_treebuild import compare_trees

    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    fills = [0xFF, 0x00, 0x7F, 0xA5]
    for i, (R, g, V, nc) in enumerate([(3, 4, 3001, 8), (1, 31, 600, 16), (6, 2, 151936, 1)]):
        print(f"[case] shared workspace outcome call {i}", flush=True)
        d = synth.pointmass_inputs(R, g, V, "bf16", T=0.9, seed=40 + i)
        ws.fill_(fills[i % 4])
        got = gpu_outcome(d, nc, workspace=ws)
        o = oracle.outcome_topk(d["target"], d["draft_tokens"], d["T"], nc, dtype="bf16",
                                want_all=True)
        compare_outcomes(got, o["all_scores"], o, f"outcome-call{i}")
        ws.fill_(fills[(i + 1) % 4])
        got = gpu_pointmass(d, workspace=ws)
        o = oracle.chain_pointmass(d["target"], d["draft_tokens"], d["uniforms"], d["T"],
                                   dtype="bf16")
        compare_chain(got, o, f"pointmass-call{i}", check_dist=False, d=d, pointmass=True)
    for i, (R, M, V, W, N, nb) in enumerate([(2, 21, 5003, 4, 3, 40), (5, 7, 300, 2, 6, 100),
                                             (1, 85, 151936, 4, 4, 64)]):
        print(f"[case] shared workspace tree-construction call {i}", flush=True)
        d = synth.treebuild_inputs(R, M, V, "bf16", T=1.0, logits=("gumbel", 2.0), seed=50 + i)
        ws.fill_(fills[(i + 2) % 4])
        par, tok, row, sc, n = sv.spec_tree_build(to_dev_logits(d["logits"], "bf16"), d["T"], W,
                                                  N, nb, workspace=ws)
        torch.cuda.synchronize()
        o = oracle.tree_build(d["logits"], d["T"], W, N, nb, dtype="bf16")
        g = dict(parents=par.cpu().numpy(), tokens=tok.cpu().numpy(), rows=row.cpu().numpy(),
                 score=sc.cpu().numpy(), n=n.cpu().numpy())
        compare_trees(g, o, nb, N, f"tree-build-call{i}", d=d, W=W)


def test_workspace_garbage_for_stochastic_trees():
    torch, sv = require_gpu()
    from gpu_util import compare_stree, to_dev, to_dev_logits

    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for i, (B, n, V, dt) in enumerate([(3, 17, 5003, "bf16"), (1, 1024, 200, "f32"),
                                       (5, 9, 151936, "bf16")]):
        print(f"[case] shared workspace stochastic-tree call {i}", flush=True)
        d = synth.stree_inputs(B, n, V, dt, T=0.8, seed=70 + i)
        ws.fill_([0xFF, 0x00, 0xA5][i])
        acc, node, out, dist = sv.spec_verify_tree_stochastic(
            to_dev_logits(d["target"], dt), to_dev_logits(d["draft"], dt),
            to_dev(d["parents"], np.int32), to_dev(d["tokens"], np.int32),
            to_dev(d["uniforms"], np.float32), d["T"], want_dist=True, workspace=ws)
        torch.cuda.synchronize()
        o = oracle.tree_stochastic(d["target"], d["draft"], d["parents"], d["tokens"],
                                   d["uniforms"], d["T"], dtype=dt, want_dist=True)
        g = dict(accept_len=acc.cpu().numpy(), accept_node=node.cpu().numpy(),
                 out_tokens=out.cpu().numpy(), final_dist=dist.cpu().numpy())
        compare_stree(g, o, f"stree-shared-ws-{i}", True, d)


def test_explicit_stream_with_binding_workspace():
    """Calls on a stream that is not the current one, with the binding's own
    outputs and cached workspace: a small call, then a larger one that grows
    the workspace (the smaller one is released while that stream may still
    use it, which the binding declares to torch's allocator), then the small
    call again.  Every result matches the oracle."""
    torch, sv = require_gpu()
    s = torch.cuda.Stream()
    small = synth.chain_inputs(3, 4, 5000, "bf16", T=0.8, seed=61)
    big = synth.chain_inputs(16, 6, 40000, "bf16", T=0.8, seed=62)
    for label, d in (("small", small), ("big", big), ("small-again", small)):
        g = gpu_chain(d, want_dist=True, stream=s)
        o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                         dtype=d["dtype"], want_dist=True)
        compare_chain(g, o, f"stream-{label}", d=d)
