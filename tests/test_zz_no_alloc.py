"""The allocation-free chain entry point (spec_verify_chain_noalloc, for
callers that cannot allocate) against spec_verify_chain with a workspace, on
the same inputs: bit-identical accept lengths and tokens and final_dist, on
two calls in a row (the second with a smaller input, which reuses the static
scratch the first left behind), and the oracle's parity rule on both."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_chain, require_gpu, to_dev, to_dev_logits

pytestmark = pytest.mark.gpu


def _both(d, want_dist):
    torch, sv = require_gpu()
    args = (to_dev_logits(d["target"], d["dtype"]), to_dev_logits(d["draft"], d["dtype"]),
            to_dev(d["draft_tokens"], np.int32), to_dev(d["uniforms"], np.float32), d["T"])
    a_acc, a_out, a_dist = sv.spec_verify_chain_noalloc(*args, want_dist=want_dist)
    torch.cuda.synchronize()
    b_acc, b_out, b_dist = sv.spec_verify_chain(*args, want_dist=want_dist)
    torch.cuda.synchronize()
    na = dict(accept_len=a_acc.cpu().numpy(), out_tokens=a_out.cpu().numpy(),
              final_dist=None if a_dist is None else a_dist.cpu().numpy())
    nb = dict(accept_len=b_acc.cpu().numpy(), out_tokens=b_out.cpu().numpy(),
              final_dist=None if b_dist is None else b_dist.cpu().numpy())
    return na, nb


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    require_gpu()
    first = synth.config_inputs(3, seed=3077)  # B=64, gamma=16, V=151936 bf16
    second = synth.chain_inputs(5, 3, 20003, "f32", T=0.9, seed=78)  # smaller, unaligned rows
    for label, d, want_dist in (("noalloc-config3", first, False),
                                ("noalloc-small", second, True)):
        print(f"[case] {label} B={d['B']} gamma={d['gamma']} V={d['V']} {d['dtype']}", flush=True)
        na, nb = _both(d, want_dist)
        assert np.array_equal(na["accept_len"], nb["accept_len"]), label
        assert np.array_equal(na["out_tokens"], nb["out_tokens"]), label
        if want_dist:
            assert np.array_equal(na["final_dist"], nb["final_dist"]), label
        o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                         dtype=d["dtype"], want_dist=want_dist)
        compare_chain(na, o, label, check_dist=want_dist, d=d)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    torch, sv = require_gpu()
    c = sv.SpecVerifyError
    B, g, V = 8192, 16, 151936
    assert sv.spec_verify_chain_workspace_bytes(B, g, V, sv.SV_DTYPE_BF16) > \
        sv.SV_NOALLOC_SCRATCH_BYTES
    # one small device tensor stands in for every input: the size check fails
    # before anything is read or enqueued
    t = torch.zeros((1, 1, 1), dtype=torch.bfloat16, device="cuda")
    lib = sv.load_library()
    import ctypes as ct

    P = ct.c_void_p(t.data_ptr())
    st = lib.spec_verify_chain_noalloc(P, P, sv.SV_DTYPE_BF16, P, P, B, g, V, 1.0, P, P, None,
                                       None)
    assert st == 8, st
    assert "scratch" in sv.spec_verify_status_string(st)
