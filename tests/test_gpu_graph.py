"""Every entry point inside a captured HIP graph (needs an MI355X).

Callers capture verification into graphs; the library allocates nothing,
records no memsets and keeps no state, so a captured call must give the
eager results on every replay.  Each case runs eagerly, is captured once,
and is replayed three times with unrelated eager work and synchronisations
in between; every replay must reproduce the eager outputs exactly."""
import numpy as np
import pytest

import synth
from gpu_util import require_gpu, to_dev, to_dev_logits

pytestmark = pytest.mark.gpu


def check_graph(run, label):
    """run() enqueues the call on the current stream and returns its output
    tensors."""
    torch, _ = require_gpu()
    print(f"[case] graph {label}", flush=True)
    eager = [t.clone() for t in run()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream (workspaces are allocated here)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        outs = run()
    for rep in range(3):
        for t in outs:
            t.fill_(-7)  # stale values must not survive a replay
        scratch = torch.randn(1 << 20, device="cuda")  # unrelated eager work in between
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a, b), f"{label}: replay {rep} differs"


def test_graph_every_entry_point():
    torch, sv = require_gpu()
    dev = torch.device("cuda")

    d = synth.chain_inputs(4, 5, 3001, "bf16", T=0.8, seed=1)
    tg, dr = to_dev_logits(d["target"], "bf16"), to_dev_logits(d["draft"], "bf16")
    tok, uni = to_dev(d["draft_tokens"], np.int32), to_dev(d["uniforms"], np.float32)
    ws = torch.empty(sv.spec_verify_chain_workspace_bytes(4, 5, 3001, sv.SV_DTYPE_BF16),
                     dtype=torch.uint8, device=dev)
    check_graph(lambda: sv.spec_verify_chain(tg, dr, tok, uni, d["T"], want_dist=True,
                                             workspace=ws), "chain")

    p = synth.pointmass_inputs(4, 5, 3001, "bf16", T=0.8, seed=2)
    ptg, ptok, puni = (to_dev_logits(p["target"], "bf16"), to_dev(p["draft_tokens"], np.int32),
                       to_dev(p["uniforms"], np.float32))
    pws = torch.empty(sv.spec_verify_chain_pointmass_workspace_bytes(4, 5, 3001,
                                                                     sv.SV_DTYPE_BF16),
                      dtype=torch.uint8, device=dev)
    check_graph(lambda: sv.spec_verify_chain_pointmass(ptg, ptok, puni, p["T"], want_dist=True,
                                                       workspace=pws), "point-mass chain")

    t = synth.tree_inputs(3, 64, 5003, seed=3)
    ttg, tpar, ttok = (to_dev_logits(t["target"], "bf16"), to_dev(t["parents"], np.int32),
                       to_dev(t["tokens"], np.int32))
    tws = torch.empty(sv.spec_verify_tree_greedy_workspace_bytes(3, 64, 5003, sv.SV_DTYPE_BF16),
                      dtype=torch.uint8, device=dev)
    check_graph(lambda: sv.spec_verify_tree_greedy(ttg, tpar, ttok, workspace=tws), "greedy tree")

    st = synth.stree_inputs(3, 33, 4001, "bf16", T=0.9, seed=4)
    stg, sdr = to_dev_logits(st["target"], "bf16"), to_dev_logits(st["draft"], "bf16")
    spar, stok, suni = (to_dev(st["parents"], np.int32), to_dev(st["tokens"], np.int32),
                        to_dev(st["uniforms"], np.float32))
    sws = torch.empty(sv.spec_verify_tree_stochastic_workspace_bytes(3, 33, 4001,
                                                                     sv.SV_DTYPE_BF16),
                      dtype=torch.uint8, device=dev)
    check_graph(lambda: sv.spec_verify_tree_stochastic(stg, sdr, spar, stok, suni, st["T"],
                                                       want_dist=True, workspace=sws)[:3],
                "stochastic tree")

    ows = torch.empty(sv.spec_outcome_topk_workspace_bytes(4, 5, 3001, sv.SV_DTYPE_BF16, 8),
                      dtype=torch.uint8, device=dev)

    def outcome_and_lookup():
        k, a, pr, hit = sv.spec_outcome_topk(ptg, ptok, p["T"], 8, workspace=ows)
        acc, out, _ = sv.spec_verify_chain_pointmass(ptg, ptok, puni, p["T"], workspace=pws)
        return k, a, pr, hit, sv.spec_cache_lookup(acc, out, k, a)

    check_graph(outcome_and_lookup, "outcome cache and lookup")

    b = synth.treebuild_inputs(3, 21, 2000, "bf16", logits=("normal", 2.0), seed=5)
    blg = to_dev_logits(b["logits"], "bf16")
    bws = torch.empty(sv.spec_tree_build_workspace_bytes(3, 21, 2000, sv.SV_DTYPE_BF16, 4, 3, 30),
                      dtype=torch.uint8, device=dev)
    check_graph(lambda: sv.spec_tree_build(blg, b["T"], 4, 3, 30, workspace=bws),
                "tree construction")


def test_graph_with_explicit_stream_and_binding_workspace():
    """The call names the capture stream explicitly and lets the binding
    provide its workspace (allocated by the warm-up call, reused under
    capture) and its outputs."""
    torch, sv = require_gpu()
    d = synth.chain_inputs(4, 5, 3001, "bf16", T=0.8, seed=121)
    tg, dr = to_dev_logits(d["target"], "bf16"), to_dev_logits(d["draft"], "bf16")
    tok, uni = to_dev(d["draft_tokens"], np.int32), to_dev(d["uniforms"], np.float32)
    check_graph(lambda: sv.spec_verify_chain(tg, dr, tok, uni, d["T"], want_dist=True,
                                             stream=torch.cuda.current_stream()),
                "chain, explicit stream")
