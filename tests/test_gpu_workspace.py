"""One scratch workspace shared by calls of different sizes and both entry
points.

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
                compare_chain(g, o, f"call{i}-dist{want_dist}")
        else:
            ws.fill_(fills[i % len(fills)])
            g = gpu_tree(dict(d, dtype="bf16"), workspace=ws)
            o = oracle.tree_greedy(d["target"], d["parents"], d["tokens"])
            compare_tree(g, o, f"call{i}")
