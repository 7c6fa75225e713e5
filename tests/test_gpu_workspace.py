"""One workspace shared by calls of different sizes and both entry points.

Every call must leave every workspace byte it used at zero (arrival counters,
row partials, chunk sums, per-block decisions), so a zero-filled workspace can
serve any later call that fits in it.  Regression test for a workspace reused
across shapes: results must match the oracle after each call and the
workspace must read back all zero."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_chain, compare_tree, gpu_chain, gpu_tree, require_gpu

pytestmark = pytest.mark.gpu


def test_workspace_reused_across_shapes_and_entry_points():
    torch, sv = require_gpu()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    calls = [
        ("chain", synth.chain_inputs(3, 1, 1, "f32", seed=1)),
        ("tree", synth.tree_inputs(4, 64, 5003, seed=2)),
        ("chain", synth.chain_inputs(9, 7, 20000, "bf16", T=0.7, seed=3)),
        ("chain", synth.chain_inputs(2, 3, 5003, "f32", seed=4)),
        ("tree", synth.tree_inputs(2, 1024, 300, seed=5)),
        ("chain", synth.chain_inputs(16, 16, 4096, "bf16", T=1.2, seed=6)),
        ("tree", synth.tree_inputs(8, 17, 1000, seed=7)),
    ]
    for i, (kind, d) in enumerate(calls):
        print(f"[case] shared workspace call {i}: {kind}", flush=True)
        if kind == "chain":
            for want_dist in (False, True):
                g = gpu_chain(d, want_dist=want_dist, workspace=ws)
                o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                                 dtype=d["dtype"], want_dist=want_dist)
                compare_chain(g, o, f"call{i}-dist{want_dist}")
                assert int(torch.count_nonzero(ws)) == 0, f"call {i} left workspace bytes set"
        else:
            g = gpu_tree(dict(d, dtype="bf16"), workspace=ws)
            o = oracle.tree_greedy(d["target"], d["parents"], d["tokens"])
            compare_tree(g, o, f"call{i}")
            assert int(torch.count_nonzero(ws)) == 0, f"call {i} left workspace bytes set"
