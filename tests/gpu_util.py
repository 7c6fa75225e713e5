"""Helpers for GPU parity tests: upload seeded inputs, call the HIP library
through its C ABI (the Python binding), and compare with the oracle.

Comparison rule for chains: accept lengths and emitted tokens must match the
oracle bit for bit, except in blocks where some decision on the oracle's path
(a ratio test or the final inverse-CDF draw) has its uniform within BAND of
the decision boundary; those blocks are excluded and counted.  The draw
distribution (final_dist) must match to DIST_TOL absolute wherever the accept
length matches.  Tree results must match exactly, with no exclusions.
"""
from __future__ import annotations

import numpy as np

BAND = 1e-6
DIST_TOL = 1e-5

# (label, blocks compared, blocks inside the boundary band) of every chain
# comparison in this session; printed at the end of the run.
RECORDS = []


def torch_mod():
    import torch

    return torch


def require_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X; none found")
    import exact_draft_verification_amd as sv

    sv.load_library()  # raises if the HIP library is not built: no fallback
    return torch, sv


def to_dev_logits(arr, dtype):
    torch = torch_mod()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).cuda()
    bits = np.ascontiguousarray(arr, np.uint16).view(np.int16)
    return torch.from_numpy(bits).cuda().view(torch.bfloat16)


def to_dev(arr, np_dtype):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(arr, np_dtype)).cuda()


def gpu_chain(d, want_dist=False, workspace=None, stream=None):
    torch, sv = require_gpu()
    tgt = to_dev_logits(d["target"], d["dtype"])
    drf = to_dev_logits(d["draft"], d["dtype"])
    tok = to_dev(d["draft_tokens"], np.int32)
    uni = to_dev(d["uniforms"], np.float32)
    acc, out, dist = sv.spec_verify_chain(tgt, drf, tok, uni, d["T"], want_dist=want_dist,
                                          workspace=workspace, stream=stream)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                final_dist=None if dist is None else dist.cpu().numpy())


def gpu_pointmass(d, want_dist=False, workspace=None, stream=None):
    torch, sv = require_gpu()
    tgt = to_dev_logits(d["target"], d["dtype"])
    tok = to_dev(d["draft_tokens"], np.int32)
    uni = to_dev(d["uniforms"], np.float32)
    acc, out, dist = sv.spec_verify_chain_pointmass(tgt, tok, uni, d["T"], want_dist=want_dist,
                                                    workspace=workspace, stream=stream)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                final_dist=None if dist is None else dist.cpu().numpy())


def gpu_tree(d, workspace=None):
    torch, sv = require_gpu()
    tgt = to_dev_logits(d["target"], d.get("dtype", "bf16"))
    par = to_dev(d["parents"], np.int32)
    tok = to_dev(d["tokens"], np.int32)
    acc, node, out = sv.spec_verify_tree_greedy(tgt, par, tok, workspace=workspace)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), accept_node=node.cpu().numpy(),
                out_tokens=out.cpu().numpy())


def compare_chain(gpu, orc, label="", check_dist=True):
    """Assert parity; return (n_compared, n_excluded)."""
    acc_g, out_g = gpu["accept_len"], gpu["out_tokens"]
    acc_o, out_o = orc["accept_len"], orc["out_tokens"]
    invalid = acc_o < 0
    near = (~invalid) & (orc["margin"] < BAND)
    cmp = ~near
    bad = np.nonzero(cmp & ((acc_g != acc_o) | (out_g != out_o).any(axis=1)))[0]
    if bad.size:
        b = bad[0]
        raise AssertionError(
            f"{label}: {bad.size} block(s) differ outside the {BAND:g} band; first b={b}: "
            f"gpu k={acc_g[b]} tokens={out_g[b].tolist()} vs oracle k={acc_o[b]} "
            f"tokens={out_o[b].tolist()} margin={orc['margin'][b]:.3g}")
    if check_dist and gpu.get("final_dist") is not None and orc.get("final_dist") is not None:
        same_k = (acc_g == acc_o) & ~invalid & (orc["fallback"] == 0)
        if same_k.any():
            err = np.abs(gpu["final_dist"][same_k].astype(np.float64) - orc["final_dist"][same_k])
            assert err.max() <= DIST_TOL, f"{label}: final_dist max abs error {err.max():.3g}"
        if invalid.any():
            assert (gpu["final_dist"][invalid] == 0).all(), f"{label}: invalid block dist not zero"
    RECORDS.append((label, int(cmp.sum()), int(near.sum())))
    return int(cmp.sum()), int(near.sum())


def compare_tree(gpu, orc, label=""):
    for key in ("accept_len", "accept_node", "out_tokens"):
        a, b = gpu[key], orc[key]
        if not np.array_equal(a, b):
            idx = np.argwhere(a != b)[0]
            raise AssertionError(f"{label}: {key} differs at {tuple(idx)}: gpu {a[tuple(idx)]} "
                                 f"vs oracle {b[tuple(idx)]}")
