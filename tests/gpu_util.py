"""Helpers for GPU parity tests: upload seeded inputs, call the HIP library
through its C ABI (the Python binding), and compare with the oracle.

Comparison rule for chains: accept lengths and emitted tokens must match the
oracle bit for bit, except in blocks where some decision on the oracle's path
(a ratio test or the final inverse-CDF draw) has its uniform within BAND of
the decision boundary.  Those blocks are counted and checked against the set
of outcomes the oracle gives with each banded uniform moved just outside the
band on either side (tests/admissible.py).  Blocks outside the library's
documented numeric domain (a row whose largest finite logit m has
|m| / T > 2^28) must come back flagged -1; they are counted apart.  The draw
distribution (final_dist) must match to DIST_TOL absolute wherever the
accept length matches.  Tree results must match exactly, with no exclusions.
"""
from __future__ import annotations

import numpy as np

import admissible

BAND = 1e-6
DIST_TOL = 1e-5

# The library's restriction on row magnitudes (include/spec_verify.h): a
# row whose largest finite logit m has |m| / T above this is outside its
# numeric domain, and the library flags that block -1.
LIB_DOMAIN = 2.0 ** 28

# One dict per comparison in this session (kind, label and counts); the
# conftest prints their totals at the end of the run.
RECORDS = []


def record(kind, label, **counts):
    RECORDS.append(dict(kind=kind, label=label, **{k: int(v) for k, v in counts.items()}))


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


def gpu_outcome(d, ncache, workspace=None):
    torch, sv = require_gpu()
    lg = to_dev_logits(d["target"], d["dtype"])
    tok = to_dev(d["draft_tokens"], np.int32)
    k, a, p, hit = sv.spec_outcome_topk(lg, tok, d["T"], ncache, workspace=workspace)
    torch.cuda.synchronize()
    return dict(k=k.cpu().numpy(), a=a.cpu().numpy(), p=p.cpu().numpy(), hit=hit.cpu().numpy())


def compare_outcomes(gpu, orc_all, orc, label="", rel=1e-6):
    """Cache parity.  orc: the oracle's cache of the same size; orc_all: its
    scores of every outcome [R, gamma+1, V].  Slot by slot the GPU must keep
    the oracle's outcome, or -- only where the two differ -- an outcome whose
    oracle probability is within `rel` of the oracle's entry (a near-tie
    whose order rounding may swap); probabilities and hit probabilities agree
    to `rel`.  Returns the number of near-tie swaps."""
    R, nc = orc["k"].shape
    swaps = 0
    for r in range(R):
        if orc["hit"][r] < 0:
            assert gpu["hit"][r] == -1.0 and (gpu["k"][r] == -1).all(), f"{label} r={r}: invalid"
            continue
        seen = set()
        for c in range(nc):
            ko, ao, po = orc["k"][r, c], orc["a"][r, c], orc["p"][r, c]
            kg, ag, pg = gpu["k"][r, c], gpu["a"][r, c], gpu["p"][r, c]
            if ko < 0:
                assert kg == -1 and ag == -1 and pg == 0.0, f"{label} r={r} c={c}: slot not empty"
                continue
            assert kg >= 0, f"{label} r={r} c={c}: gpu slot empty, oracle {ko, ao, po}"
            assert (kg, ag) not in seen, f"{label} r={r}: duplicate {kg, ag}"
            seen.add((kg, ag))
            if (kg, ag) != (ko, ao):
                pog = orc_all[r, kg, ag]
                assert abs(pog - po) <= rel * po, (
                    f"{label} r={r} c={c}: gpu {(kg, ag)} (oracle p {pog:.12g}) vs oracle "
                    f"{(ko, ao)} p {po:.12g}")
                swaps += 1
            assert abs(pg - orc_all[r, kg, ag]) <= rel * orc_all[r, kg, ag], f"{label} r={r} c={c}: p"
        assert abs(gpu["hit"][r] - orc["hit"][r]) <= rel * orc["hit"][r], f"{label} r={r}: hit"
    record("outcome", label, requests=R, slots=int((orc["k"] >= 0).sum()), swaps=swaps)
    return swaps


def gpu_tree(d, workspace=None):
    torch, sv = require_gpu()
    tgt = to_dev_logits(d["target"], d.get("dtype", "bf16"))
    par = to_dev(d["parents"], np.int32)
    tok = to_dev(d["tokens"], np.int32)
    acc, node, out = sv.spec_verify_tree_greedy(tgt, par, tok, workspace=workspace)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), accept_node=node.cpu().numpy(),
                out_tokens=out.cpu().numpy())


def _decoded(arr, dtype):
    a = np.asarray(arr)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def outside_domain(d, pointmass=False):
    """[B] bool: blocks with a row outside the library's numeric domain."""
    T = float(d["T"])
    keys = ("target",) if pointmass else ("target", "draft")
    out = np.zeros(d["target"].shape[0], bool)
    for key in keys:
        z = _decoded(d[key], d["dtype"])
        with np.errstate(invalid="ignore"):
            fin = np.where(np.isfinite(z), z, -np.inf)
            m = fin.max(axis=2)
        big = np.isfinite(m) & (np.abs(m.astype(np.float64)) / T > LIB_DOMAIN)
        out |= big.any(axis=1)
    return out


def compare_chain(gpu, orc, label="", check_dist=True, d=None, pointmass=False):
    """Assert parity of a chain (or point-mass chain) call.  d holds the
    inputs (needed for the band and domain checks).  Returns
    (n_compared_exactly, n_in_band)."""
    acc_g, out_g = gpu["accept_len"], gpu["out_tokens"]
    acc_o, out_o = orc["accept_len"], orc["out_tokens"]
    invalid = acc_o < 0
    dom = np.zeros_like(invalid)
    if d is not None:
        dom = outside_domain(d, pointmass) & ~invalid
    if dom.any():
        assert (acc_g[dom] == -1).all() and (out_g[dom] == -1).all(), (
            f"{label}: a block outside the library's domain was not flagged -1")
    near = (~invalid) & (~dom) & (orc["margin"] < BAND)
    cmp = ~near & ~dom
    bad = np.nonzero(cmp & ((acc_g != acc_o) | (out_g != out_o).any(axis=1)))[0]
    if bad.size:
        b = bad[0]
        raise AssertionError(
            f"{label}: {bad.size} block(s) differ outside the {BAND:g} band; first b={b}: "
            f"gpu k={acc_g[b]} tokens={out_g[b].tolist()} vs oracle k={acc_o[b]} "
            f"tokens={out_o[b].tolist()} margin={orc['margin'][b]:.3g}")
    nb = np.nonzero(near)[0]
    if nb.size:
        assert d is not None, f"{label}: {nb.size} banded block(s) need the inputs to be checked"
        for b in nb:
            leaves = admissible.chain_leaves(
                d["target"][b], None if pointmass else d["draft"][b], d["draft_tokens"][b],
                d["uniforms"][b], d["T"], d["dtype"], pointmass=pointmass)
            assert admissible.matches(leaves, int(acc_g[b]), out_g[b]), (
                f"{label}: banded block b={b}: gpu k={acc_g[b]} tokens={out_g[b].tolist()} is "
                f"not among the admissible outcomes {admissible.describe(leaves)}")
    if check_dist and gpu.get("final_dist") is not None and orc.get("final_dist") is not None:
        same_k = (acc_g == acc_o) & ~invalid & ~dom & (orc["fallback"] == 0)
        if same_k.any():
            err = np.abs(gpu["final_dist"][same_k].astype(np.float64) - orc["final_dist"][same_k])
            assert err.max() <= DIST_TOL, f"{label}: final_dist max abs error {err.max():.3g}"
        if invalid.any():
            assert (gpu["final_dist"][invalid] == 0).all(), f"{label}: invalid block dist not zero"
    record("pointmass" if pointmass else "chain", label, exact=cmp.sum(), band_checked=nb.size,
           domain=dom.sum(), invalid=invalid.sum())
    return int(cmp.sum()), int(near.sum())


def compare_tree(gpu, orc, label=""):
    for key in ("accept_len", "accept_node", "out_tokens"):
        a, b = gpu[key], orc[key]
        if not np.array_equal(a, b):
            idx = np.argwhere(a != b)[0]
            raise AssertionError(f"{label}: {key} differs at {tuple(idx)}: gpu {a[tuple(idx)]} "
                                 f"vs oracle {b[tuple(idx)]}")
    record("tree_greedy", label, exact=len(orc["accept_len"]))


def compare_stree(g, o, label, want_dist, d):
    """Stochastic tree parity: exact outputs outside the boundary band; a
    request with a decision inside it (a node test under an accepted parent,
    or the draw) must give one of the oracle's admissible outcomes; -1 for
    invalid requests; final_dist to DIST_TOL where the draw's node is the
    same."""
    bad = o["accept_len"] < 0  # invalid requests: -1 everywhere on both sides
    assert (g["accept_len"][bad] == -1).all() and (g["accept_node"][bad] == -1).all()
    assert (g["out_tokens"][bad] == -1).all()
    keep = (o["margin"] >= BAND) & ~bad
    for key in ("accept_len", "accept_node", "out_tokens"):
        assert np.array_equal(g[key][keep], o[key][keep]), f"{label}: {key}"
    near = np.nonzero(~keep & ~bad)[0]
    for b in near:
        leaves = admissible.stree_leaves(d["target"][b], d["draft"][b], d["parents"][b],
                                         d["tokens"][b], d["uniforms"][b], d["T"], d["dtype"])
        assert admissible.matches(leaves, int(g["accept_len"][b]), g["out_tokens"][b]), (
            f"{label}: banded request b={b}: gpu k={g['accept_len'][b]} "
            f"tokens={g['out_tokens'][b].tolist()} not among {admissible.describe(leaves)}")
    if want_dist:
        same = (g["accept_node"] == o["accept_node"]) & (o["accept_len"] >= 0)
        if same.any():
            err = np.abs(g["final_dist"][same] - o["final_dist"][same]).max()
            assert err <= DIST_TOL, f"{label}: final_dist differs by {err}"
        assert (g["final_dist"][bad] == 0).all()
    record("tree_stochastic", label, exact=keep.sum(), band_checked=near.size, invalid=bad.sum())
    print(f"[case] {label}: compared {int(keep.sum())}, in band {near.size} (checked), "
          f"invalid {int(bad.sum())}", flush=True)

