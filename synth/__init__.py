"""Seeded synthetic inputs for speculative-decoding verification.

This module only *draws* inputs: logits, draft tokens, draft-tree parent arrays
and the uniforms that drive every random decision of the verifier.  It holds
none of the verifier's arithmetic (no softmax, ratio test, residual or greedy
path logic), so the oracle and the HIP path can both be fed from it without
sharing any part of what they compute.

Workload shapes follow the statement of the problem on the pages: a chain
block has gamma draft positions and gamma+1 target rows, the last one being
the bonus row ("JetSpec++", Appendix F.1 / Proposition 1; "Speculative
decoding verifies draft tokens ...", section "A fully accepted block yields
more than one committed token"); a draft tree is a parent array whose node 0
is the root ("JetSpec reading notes", Algorithm 1 and Fig. 3).

Recipes (all reproducible from ``seed``; each block or request draws from its
own child stream of ``numpy.random.SeedSequence(seed)`` so blocks can be drawn
in parallel threads without changing the result):

* chain, per block: target rows ``[gamma+1, V]`` (normal or Gumbel, scaled),
  optional "boost" of ``count`` distinct token ids per target row, draft rows
  ``target[i] + N(0, noise^2)`` for ``i < gamma``; both rounded to the storage
  dtype (fp32, or bf16 by round-to-nearest-even); draft token ``d_i`` sampled
  from ``softmax(draft_i / T)`` with the Gumbel-max trick; uniforms
  ``U[0,1)`` float32 of shape ``[gamma+1]``.
* tree, per request: parent array with depth and branching caps, node rows
  i.i.d. ``N(0, sigma^2)`` whose maximum is planted at a known position (the
  maximum is drawn from its exact distribution and the other entries
  conditioned below it), tokens equal to the parent's planted maximum with
  probability ``p_match`` and uniform otherwise.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os as _os

import numpy as np

__all__ = [
    "CONFIGS",
    "POINTMASS_CONFIGS",
    "pointmass_inputs",
    "pointmass_config_inputs",
    "pointmass_config_bytes",
    "OUTCOME_CONFIG",
    "outcome_config_inputs",
    "outcome_config_bytes",
    "bf16_bits",
    "bf16_to_f32",
    "chain_inputs",
    "tree_inputs",
    "config_inputs",
    "config_bytes",
    "redraw_chain_tokens",
]

# The five workloads: sizes, distributions and temperatures.  V = 151936 is a
# Qwen3-sized vocabulary (the pages evaluate Qwen3-8B but never state V).
CONFIGS = {
    1: dict(kind="chain", B=1, gamma=4, V=1024, dtype="f32", T=1.0,
            target=("normal", 2.0), noise=0.5, boost=None),
    2: dict(kind="chain", B=1, gamma=16, V=151936, dtype="f32", T=1.0,
            target=("gumbel", 3.0), noise=0.7, boost=None),
    3: dict(kind="chain", B=64, gamma=16, V=151936, dtype="bf16", T=0.7,
            target=("normal", 2.5), noise=1.0, boost=(5, 8.0)),
    4: dict(kind="tree", B=64, n=64, V=151936, dtype="bf16", sigma=2.0,
            max_depth=16, max_children=4, p_match=0.8),
    5: dict(kind="chain", B=256, gamma=16, V=151936, dtype="bf16", T=0.6,
            target=("gumbel", 4.0), noise=0.8, boost=None),
}

_U24 = np.float32(2.0 ** -24)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN stays NaN (quiet), +-inf stay
    +-inf, finite values that round past the largest bf16 become +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gumbel(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard Gumbel(0, 1) draws in float32.

    Uniforms are taken on the open grid {k * 2^-24 : 1 <= k < 2^24} so both
    logarithms stay finite; the upper tail is therefore truncated near 16.6.
    """
    k = rng.integers(1, 1 << 24, size=shape, dtype=np.int32)
    u = k.astype(np.float32) * _U24
    return -np.log(-np.log(u))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _as_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    return stored if dtype == "f32" else bf16_to_f32(stored)


def _workers(n_items: int, threads: int | None) -> int:
    if threads is None:
        threads = min(16, _os.cpu_count() or 1)
    return max(1, min(threads, n_items))


def _chain_block(seed_seq, gamma, V, dtype, T, target, noise, boost):
    rng = np.random.default_rng(seed_seq)
    kind, scale = target
    if kind == "normal":
        t = rng.standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(scale)
    elif kind == "gumbel":
        t = _gumbel(rng, (gamma + 1, V)) * np.float32(scale)
    else:
        raise ValueError(f"unknown target distribution {kind!r}")
    if boost is not None:
        count, amount = boost
        for j in range(gamma + 1):
            ids = rng.choice(V, size=count, replace=False)
            t[j, ids] += np.float32(amount)
    t_st = _store(t, dtype)
    t_val = _as_f32(t_st, dtype)
    d = t_val[:gamma] + rng.standard_normal((gamma, V), dtype=np.float32) * np.float32(noise)
    d_st = _store(d, dtype)
    d_val = _as_f32(d_st, dtype)
    # Gumbel-max: argmax_v (z_v / T + G_v) is an exact draw from softmax(z / T).
    g = _gumbel(rng, (gamma, V))
    tokens = np.argmax(d_val / np.float32(T) + g, axis=1).astype(np.int32)
    u = rng.random(gamma + 1, dtype=np.float32)
    return t_st, d_st, tokens, u


def chain_inputs(B: int, gamma: int, V: int, dtype: str = "f32", T: float = 1.0,
                 target=("normal", 2.0), noise: float = 0.5, boost=None,
                 seed: int = 0, threads: int | None = None) -> dict:
    """Inputs for one chain-verification call.

    Returns a dict with ``target`` [B, gamma+1, V] and ``draft`` [B, gamma, V]
    (float32 arrays, or uint16 bf16 bit patterns), ``draft_tokens`` int32
    [B, gamma], ``uniforms`` float32 [B, gamma+1] (entry i < gamma drives the
    test at draft position i, entry gamma the final draw), and the scalars.
    """
    if B < 1 or gamma < 1 or V < 1:
        raise ValueError("B, gamma and V must be >= 1")
    st = np.uint16 if dtype == "bf16" else np.float32
    tgt = np.empty((B, gamma + 1, V), dtype=st)
    drf = np.empty((B, gamma, V), dtype=st)
    tok = np.empty((B, gamma), dtype=np.int32)
    uni = np.empty((B, gamma + 1), dtype=np.float32)
    children = np.random.SeedSequence(seed).spawn(B)

    def work(b):
        tgt[b], drf[b], tok[b], uni[b] = _chain_block(
            children[b], gamma, V, dtype, T, target, noise, boost)

    nw = _workers(B, threads)
    if nw == 1:
        for b in range(B):
            work(b)
    else:
        with _cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, range(B)))
    return dict(kind="chain", target=tgt, draft=drf, draft_tokens=tok, uniforms=uni,
                B=B, gamma=gamma, V=V, dtype=dtype, T=float(T))


# Point-mass ("exact-match") chain workloads: the shapes and target logits of
# chain configurations 3 and 5, no draft logits, and draft tokens that equal
# the target row's argmax with probability p_match (a greedy draft that
# agrees with the target most of the time), else a uniform token.
POINTMASS_CONFIGS = {
    3: dict(B=64, gamma=16, V=151936, dtype="bf16", T=0.7, target=("normal", 2.5),
            boost=(5, 8.0), p_match=0.8),
    5: dict(B=256, gamma=16, V=151936, dtype="bf16", T=0.6, target=("gumbel", 4.0),
            boost=None, p_match=0.8),
}


def _pointmass_block(seed_seq, gamma, V, dtype, target, boost, p_match):
    rng = np.random.default_rng(seed_seq)
    kind, scale = target
    if kind == "normal":
        t = rng.standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(scale)
    elif kind == "gumbel":
        t = _gumbel(rng, (gamma + 1, V)) * np.float32(scale)
    else:
        raise ValueError(f"unknown target distribution {kind!r}")
    if boost is not None:
        count, amount = boost
        for j in range(gamma + 1):
            ids = rng.choice(V, size=count, replace=False)
            t[j, ids] += np.float32(amount)
    t_st = _store(t, dtype)
    amax = np.argmax(_as_f32(t_st, dtype)[:gamma], axis=1)
    match = rng.random(gamma) < p_match
    other = rng.integers(0, V, gamma)
    tokens = np.where(match, amax, other).astype(np.int32)
    u = rng.random(gamma + 1, dtype=np.float32)
    return t_st, tokens, u


def pointmass_inputs(B: int, gamma: int, V: int, dtype: str = "f32", T: float = 1.0,
                     target=("normal", 2.0), boost=None, p_match: float = 0.8, seed: int = 0,
                     threads: int | None = None) -> dict:
    """Inputs for one point-mass chain call: ``target`` [B, gamma+1, V],
    ``draft_tokens`` int32 [B, gamma] (the target row's argmax with
    probability p_match, else uniform), ``uniforms`` float32 [B, gamma+1]."""
    if B < 1 or gamma < 1 or V < 1:
        raise ValueError("B, gamma and V must be >= 1")
    st = np.uint16 if dtype == "bf16" else np.float32
    tgt = np.empty((B, gamma + 1, V), dtype=st)
    tok = np.empty((B, gamma), dtype=np.int32)
    uni = np.empty((B, gamma + 1), dtype=np.float32)
    children = np.random.SeedSequence(seed).spawn(B)

    def work(b):
        tgt[b], tok[b], uni[b] = _pointmass_block(children[b], gamma, V, dtype, target, boost,
                                                  p_match)

    nw = _workers(B, threads)
    if nw == 1:
        for b in range(B):
            work(b)
    else:
        with _cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, range(B)))
    return dict(kind="pointmass", target=tgt, draft_tokens=tok, uniforms=uni, B=B, gamma=gamma,
                V=V, dtype=dtype, T=float(T))


def pointmass_config_inputs(cfg: int, seed: int = 0, threads: int | None = None,
                            **overrides) -> dict:
    """Inputs for a point-mass workload with the shape of chain config cfg."""
    c = dict(POINTMASS_CONFIGS[cfg])
    c.update(overrides)
    return pointmass_inputs(c["B"], c["gamma"], c["V"], c["dtype"], c["T"], c["target"],
                            c["boost"], c["p_match"], seed=seed, threads=threads)


def pointmass_config_bytes(cfg: int, **overrides) -> int:
    """Algorithmic logit bytes of one point-mass call: every target logit once."""
    c = dict(POINTMASS_CONFIGS[cfg])
    c.update(overrides)
    e = 4 if c["dtype"] == "f32" else 2
    return c["B"] * (c["gamma"] + 1) * c["V"] * e


# Outcome scoring workload: 32 requests (the request count of config 5, whose
# 8 anticipated outcomes per request are what this scoring selects), decoder
# rows with config 5's logits and temperature, draft tokens as for the
# point-mass workloads, and a cache of 8 outcomes per request.
OUTCOME_CONFIG = dict(R=32, gamma=16, V=151936, dtype="bf16", T=0.6, target=("gumbel", 4.0),
                      boost=None, p_match=0.8, ncache=8)


def outcome_config_inputs(seed: int = 0, threads: int | None = None, **overrides) -> dict:
    """Decoder logits [R, gamma+1, V] and draft tokens [R, gamma] for the
    outcome-scoring workload (uniforms are drawn but unused)."""
    c = dict(OUTCOME_CONFIG)
    c.update(overrides)
    d = pointmass_inputs(c["R"], c["gamma"], c["V"], c["dtype"], c["T"], c["target"], c["boost"],
                         c["p_match"], seed=seed, threads=threads)
    d.update(kind="outcome", R=c["R"], ncache=c["ncache"])
    return d


def outcome_config_bytes(**overrides) -> int:
    """Algorithmic logit bytes of one outcome-scoring call."""
    c = dict(OUTCOME_CONFIG)
    c.update(overrides)
    e = 4 if c["dtype"] == "f32" else 2
    return c["R"] * (c["gamma"] + 1) * c["V"] * e


# Draft-tree construction: one row of draft logits per potential node of a
# complete W-ary tree above depth N, so M = 1 + W + ... + W^(N-1) rows.
TREEBUILD_CONFIG = dict(R=32, W=4, N=4, budget=64, V=151936, dtype="bf16", T=1.0,
                        logits=("gumbel", 3.0))


def complete_tree_rows(W: int, N: int) -> int:
    """Rows of the potential nodes above depth N in a complete W-ary tree."""
    return sum(W ** d for d in range(N))


def _treebuild_request(seed_seq, M, V, dtype, logits):
    rng = np.random.default_rng(seed_seq)
    kind, scale = logits
    if kind == "normal":
        z = rng.standard_normal((M, V), dtype=np.float32) * np.float32(scale)
    elif kind == "gumbel":
        z = _gumbel(rng, (M, V)) * np.float32(scale)
    else:
        raise ValueError(f"unknown logit distribution {kind!r}")
    return _store(z, dtype)


def treebuild_inputs(R: int, M: int, V: int, dtype: str = "f32", T: float = 1.0,
                     logits=("normal", 2.0), seed: int = 0, threads: int | None = None) -> dict:
    """Draft logits [R, M, V] for tree construction: independent rows, one per
    potential node."""
    if R < 1 or M < 1 or V < 1:
        raise ValueError("R, M and V must be >= 1")
    st = np.uint16 if dtype == "bf16" else np.float32
    z = np.empty((R, M, V), dtype=st)
    children = np.random.SeedSequence(seed).spawn(R)

    def work(r):
        z[r] = _treebuild_request(children[r], M, V, dtype, logits)

    nw = _workers(R, threads)
    if nw == 1:
        for r in range(R):
            work(r)
    else:
        with _cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, range(R)))
    return dict(kind="treebuild", logits=z, R=R, M=M, V=V, dtype=dtype, T=float(T))


def treebuild_config_inputs(seed: int = 0, threads: int | None = None, **overrides) -> dict:
    """The tree-construction workload: R requests, width W, depth N, budget."""
    c = dict(TREEBUILD_CONFIG)
    c.update(overrides)
    M = complete_tree_rows(c["W"], c["N"])
    d = treebuild_inputs(c["R"], M, c["V"], c["dtype"], c["T"], c["logits"], seed=seed,
                         threads=threads)
    d.update(W=c["W"], N=c["N"], budget=c["budget"])
    return d


def treebuild_config_bytes(**overrides) -> int:
    """Algorithmic logit bytes of one tree-construction call."""
    c = dict(TREEBUILD_CONFIG)
    c.update(overrides)
    e = 4 if c["dtype"] == "f32" else 2
    return c["R"] * complete_tree_rows(c["W"], c["N"]) * c["V"] * e


def _tree_parents(rng, n, max_depth, max_children):
    parents = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    nchild = np.zeros(n, dtype=np.int32)
    for j in range(1, n):
        ok = np.nonzero((depth[:j] < max_depth) & (nchild[:j] < max_children))[0]
        if ok.size == 0:
            raise ValueError("tree caps leave no eligible parent; raise max_depth or max_children")
        p = int(ok[rng.integers(ok.size)])
        parents[j] = p
        depth[j] = depth[p] + 1
        nchild[p] += 1
    return parents


def _planted_row(rng, V, sigma):
    """One row of V i.i.d. N(0, sigma^2) values and the position of its maximum.

    The maximum M has CDF Phi(x / sigma)^V, so M = sigma * Phi^-1(U^(1/V));
    the other V-1 entries are N(0, sigma^2) conditioned on being below M
    (rejection: redraw the few that land at or above M).  Placing M at a
    uniformly random position gives exactly an i.i.d. row whose argmax
    position is known without searching for it.
    """
    from scipy.special import ndtri

    u = max(rng.random(), 1e-300)
    # 1 - U^(1/V), computed without cancellation
    tail = -np.expm1(np.log(u) / V)
    top = -float(ndtri(tail)) * sigma
    row = rng.standard_normal(V, dtype=np.float32) * np.float32(sigma)
    w = int(rng.integers(V))
    while True:
        bad = np.nonzero(row >= np.float32(top))[0]
        bad = bad[bad != w]
        if bad.size == 0:
            break
        row[bad] = rng.standard_normal(bad.size, dtype=np.float32) * np.float32(sigma)
    row[w] = np.float32(top)
    return row, w


def _tree_request(seed_seq, n, V, sigma, max_depth, max_children, p_match):
    rng = np.random.default_rng(seed_seq)
    parents = _tree_parents(rng, n, max_depth, max_children)
    rows = np.empty((n, V), dtype=np.uint16)
    planted = np.empty(n, dtype=np.int64)
    for j in range(n):
        r, w = _planted_row(rng, V, sigma)
        rows[j] = bf16_bits(r)
        planted[j] = w
    tokens = np.zeros(n, dtype=np.int32)
    for j in range(1, n):
        if rng.random() < p_match:
            tokens[j] = planted[parents[j]]
        else:
            tokens[j] = rng.integers(V)
    return rows, parents, tokens


def tree_inputs(B: int, n: int, V: int, sigma: float = 2.0, max_depth: int = 16,
                max_children: int = 4, p_match: float = 0.8, seed: int = 0,
                threads: int | None = None) -> dict:
    """Inputs for one greedy tree-verification call (bf16 logits).

    ``target`` [B, n, V] uint16 bf16 bits, row j = target logits after the
    root->j path; ``parents`` int32 [B, n] with parents[0] = -1 and
    0 <= parents[j] < j; ``tokens`` int32 [B, n] (tokens[0] is the anchor and
    is never checked).  After bf16 rounding a row may hold ties for its
    maximum; the planted position is then one of the tied entries.
    """
    if B < 1 or n < 1 or V < 1:
        raise ValueError("B, n and V must be >= 1")
    tgt = np.empty((B, n, V), dtype=np.uint16)
    par = np.empty((B, n), dtype=np.int32)
    tok = np.empty((B, n), dtype=np.int32)
    children = np.random.SeedSequence(seed).spawn(B)

    def work(b):
        tgt[b], par[b], tok[b] = _tree_request(children[b], n, V, sigma, max_depth,
                                               max_children, p_match)

    nw = _workers(B, threads)
    if nw == 1:
        for b in range(B):
            work(b)
    else:
        with _cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, range(B)))
    return dict(kind="tree", target=tgt, parents=par, tokens=tok, B=B, n=n, V=V,
                dtype="bf16")


# Stochastic tree verification: config 4's trees with draft logits per node
# and node tokens drawn from the draft at their parent.
STREE_CONFIG = dict(B=64, n=64, V=151936, dtype="bf16", T=1.0, target=("normal", 2.0),
                    noise=1.0, max_depth=16, max_children=4)


def _stree_request(seed_seq, n, V, dtype, T, target, noise, max_depth, max_children):
    rng = np.random.default_rng(seed_seq)
    parents = _tree_parents(rng, n, max_depth, max_children)
    kind, scale = target
    if kind == "normal":
        t = rng.standard_normal((n, V), dtype=np.float32) * np.float32(scale)
    elif kind == "gumbel":
        t = _gumbel(rng, (n, V)) * np.float32(scale)
    else:
        raise ValueError(f"unknown target distribution {kind!r}")
    d = t + rng.standard_normal((n, V), dtype=np.float32) * np.float32(noise)
    t_st, d_st = _store(t, dtype), _store(d, dtype)
    # node j's token ~ q at its parent (Gumbel-max over the stored draft row)
    dq = _as_f32(d_st, dtype).astype(np.float64) / T
    tokens = np.zeros(n, dtype=np.int32)
    for j in range(1, n):
        tokens[j] = int(np.argmax(dq[parents[j]] + _gumbel(rng, V)))
    u = rng.random(n, dtype=np.float32)
    return t_st, d_st, parents, tokens, u


def stree_inputs(B: int, n: int, V: int, dtype: str = "bf16", T: float = 1.0,
                 target=("normal", 2.0), noise: float = 1.0, max_depth: int = 16,
                 max_children: int = 4, seed: int = 0, threads: int | None = None) -> dict:
    """Inputs for one stochastic tree-verification call: ``target`` and
    ``draft`` [B, n, V] (row j = logits after node j's path), ``parents`` and
    ``tokens`` int32 [B, n] (node tokens drawn from the draft at their
    parent), ``uniforms`` float32 [B, n]."""
    if B < 1 or n < 1 or V < 1:
        raise ValueError("B, n and V must be >= 1")
    st = np.uint16 if dtype == "bf16" else np.float32
    tgt = np.empty((B, n, V), dtype=st)
    drf = np.empty((B, n, V), dtype=st)
    par = np.empty((B, n), dtype=np.int32)
    tok = np.empty((B, n), dtype=np.int32)
    uni = np.empty((B, n), dtype=np.float32)
    children = np.random.SeedSequence(seed).spawn(B)

    def work(b):
        tgt[b], drf[b], par[b], tok[b], uni[b] = _stree_request(
            children[b], n, V, dtype, T, target, noise, max_depth, max_children)

    nw = _workers(B, threads)
    if nw == 1:
        for b in range(B):
            work(b)
    else:
        with _cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, range(B)))
    return dict(kind="stree", target=tgt, draft=drf, parents=par, tokens=tok, uniforms=uni, B=B,
                n=n, V=V, dtype=dtype, T=float(T))


def stree_config_inputs(seed: int = 0, threads: int | None = None, **overrides) -> dict:
    c = dict(STREE_CONFIG)
    c.update(overrides)
    return stree_inputs(c["B"], c["n"], c["V"], c["dtype"], c["T"], c["target"], c["noise"],
                        c["max_depth"], c["max_children"], seed=seed, threads=threads)


def stree_config_bytes(**overrides) -> int:
    """Algorithmic logit bytes of one stochastic tree call (target and draft)."""
    c = dict(STREE_CONFIG)
    c.update(overrides)
    e = 4 if c["dtype"] == "f32" else 2
    return 2 * c["B"] * c["n"] * c["V"] * e


def redraw_chain_tokens(d: dict, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Fresh draft tokens and uniforms for the logits of chain inputs d:
    d_i ~ softmax(draft_i / T) by the Gumbel-max trick over the stored draft
    logits, as chain_inputs draws them, and U[0, 1) float32 uniforms.
    Returns (draft_tokens [B, gamma] int32, uniforms [B, gamma+1] float32)."""
    rng = np.random.default_rng(seed)
    B, g = d["draft_tokens"].shape
    dv = _as_f32(d["draft"], d["dtype"])
    tok = np.empty((B, g), np.int32)
    for b in range(B):
        gum = _gumbel(rng, dv.shape[1:])
        tok[b] = np.argmax(dv[b] / np.float32(d["T"]) + gum, axis=1)
    return tok, rng.random((B, g + 1), dtype=np.float32)


def config_inputs(cfg: int, seed: int = 0, threads: int | None = None, **overrides) -> dict:
    """Inputs for one of the five workloads, with optional shape overrides."""
    c = dict(CONFIGS[cfg])
    c.update(overrides)
    kind = c.pop("kind")
    if kind == "chain":
        return chain_inputs(c["B"], c["gamma"], c["V"], c["dtype"], c["T"], c["target"],
                            c["noise"], c["boost"], seed=seed, threads=threads)
    return tree_inputs(c["B"], c["n"], c["V"], c["sigma"], c["max_depth"],
                       c["max_children"], c["p_match"], seed=seed, threads=threads)


def config_bytes(cfg: int, **overrides) -> int:
    """Algorithmic logit bytes of one call: every input logit read once."""
    c = dict(CONFIGS[cfg])
    c.update(overrides)
    e = 4 if c["dtype"] == "f32" else 2
    if c["kind"] == "chain":
        return c["B"] * (2 * c["gamma"] + 1) * c["V"] * e
    return c["B"] * c["n"] * c["V"] * e
