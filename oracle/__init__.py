"""ctypes front end of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only callers.  It shares no code with the GPU library
and is never a fallback for it.
"""
from __future__ import annotations

import ctypes as _ct
import os as _os
import subprocess as _sp

import numpy as np

_HERE = _os.path.dirname(_os.path.abspath(__file__))
_SRC = _os.path.join(_HERE, "oracle.c")
_LIB = _os.path.join(_HERE, "liboracle.so")
# A different build of oracle.c (for instance one with a mistake planted on
# purpose, to check that the pins in the test suite catch it) can be loaded
# instead by naming it here.
_LIB_OVERRIDE = _os.environ.get("SPEC_ORACLE_LIB")

F32, BF16 = 0, 1
_DT = {"f32": F32, "bf16": BF16}


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with plain gcc (no fast-math)."""
    if force or not _os.path.exists(_LIB) or _os.path.getmtime(_LIB) < _os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        _sp.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                        "-fno-fast-math", "-o", tmp, _SRC, "-lm", "-lpthread"])
        _os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None and _LIB_OVERRIDE:
        _lib = _declare(_ct.CDLL(_LIB_OVERRIDE))
    if _lib is None:
        if not _os.path.exists(_LIB) or _os.path.getmtime(_LIB) < _os.path.getmtime(_SRC):
            build(force=True)
        _lib = _declare(_ct.CDLL(_LIB))
    return _lib


def _declare(lib):
    P, I, D = _ct.c_void_p, _ct.c_int, _ct.c_double
    lib.oracle_chain.argtypes = [P, P, I, P, P, I, I, I, D, P, P, P, P, P, P, I]
    lib.oracle_chain_du.argtypes = [P, P, I, P, P, I, I, I, D, P, P, P, P, P, P, I]
    lib.oracle_chain_alpha.argtypes = [P, P, I, I, I, I, D, P, I]
    lib.oracle_tree_greedy.argtypes = [P, I, P, P, I, I, I, P, P, P, P, I]
    lib.oracle_chain_pointmass.argtypes = [P, I, P, P, I, I, I, D, P, P, P, P, P, P, I]
    lib.oracle_chain_pointmass_du.argtypes = [P, I, P, P, I, I, I, D, P, P, P, P, P, P, I]
    lib.oracle_outcome_topk.argtypes = [P, I, P, I, I, I, D, I, P, P, P, P, P]
    lib.oracle_tree_build.argtypes = [P, I, I, I, I, D, I, I, I, P, P, P, P, P, P, P]
    lib.oracle_tree_score.argtypes = [P, I, I, I, I, D, I, P, P, P, P, P]
    lib.oracle_tree_stochastic.argtypes = [P, P, I, P, P, P, I, I, I, D, P, P, P, P, P, P]
    lib.oracle_tree_stochastic_du.argtypes = [P, P, I, P, P, P, I, I, I, D, P, P, P, P, P, P]
    for f in (lib.oracle_chain, lib.oracle_chain_du, lib.oracle_chain_alpha,
              lib.oracle_tree_greedy, lib.oracle_chain_pointmass, lib.oracle_chain_pointmass_du,
              lib.oracle_outcome_topk, lib.oracle_tree_build, lib.oracle_tree_stochastic,
              lib.oracle_tree_stochastic_du, lib.oracle_tree_score):
        f.restype = I
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_ct.c_void_p)


def _logits(a, dtype):
    want = np.uint16 if dtype == "bf16" else np.float32
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"{dtype} logits must be stored as {np.dtype(want).name}, got {a.dtype}")
    return a


def default_threads() -> int:
    return max(1, min(16, _os.cpu_count() or 1))


def chain(target, draft, draft_tokens, uniforms, T, dtype="f32", want_dist=False,
          threads=None) -> dict:
    """Chain verification (ratio test, first rejection, residual or bonus draw).

    ``uniforms`` float32 [B, gamma+1] use the library's interface; float64
    uniforms are taken as given (continuous-u enumeration in the tests).
    Returns accept_len [B], out_tokens [B, gamma+1], margin [B] (distance of
    the nearest decision on the path to its boundary, in u units), ratios
    [B, gamma], fallback [B] and, if asked, final_dist [B, V] (the normalised
    residual, or p at the bonus row).
    """
    lib = _load()
    target = _logits(target, dtype)
    draft = _logits(draft, dtype)
    B, g1, V = target.shape
    g = g1 - 1
    if draft.shape != (B, g, V):
        raise ValueError("draft must be [B, gamma, V]")
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, g)
    u = np.ascontiguousarray(uniforms)
    if u.shape != (B, g + 1):
        raise ValueError("uniforms must be [B, gamma+1]")
    acc = np.empty(B, np.int32)
    out = np.empty((B, g + 1), np.int32)
    margin = np.empty(B, np.float64)
    ratios = np.empty((B, g), np.float64)
    fb = np.empty(B, np.int32)
    dist = np.empty((B, V), np.float64) if want_dist else None
    nt = default_threads() if threads is None else threads
    if u.dtype == np.float64:
        rc = lib.oracle_chain_du(_ptr(target), _ptr(draft), _DT[dtype], _ptr(tok), _ptr(u), B,
                                 g, V, float(T), _ptr(acc), _ptr(out), _ptr(dist),
                                 _ptr(margin), _ptr(ratios), _ptr(fb), nt)
    else:
        u = np.ascontiguousarray(u, dtype=np.float32)
        rc = lib.oracle_chain(_ptr(target), _ptr(draft), _DT[dtype], _ptr(tok), _ptr(u), B, g,
                              V, float(T), _ptr(acc), _ptr(out), _ptr(dist), _ptr(margin),
                              _ptr(ratios), _ptr(fb), nt)
    if rc != 0:
        raise ValueError(f"oracle_chain rejected its arguments (rc={rc})")
    return dict(accept_len=acc, out_tokens=out, margin=margin, ratios=ratios, fallback=fb,
                final_dist=dist)


def chain_pointmass(target, draft_tokens, uniforms, T, dtype="f32", want_dist=False,
                    threads=None) -> dict:
    """Point-mass chain verification: the draft proposes each token with
    certainty, so test i accepts with probability p_i(x_i); a rejection draws
    from p_k without x_k, renormalised; a full block draws the bonus from
    p_gamma.  Same outputs as ``chain`` (``ratios`` hold p_i(x_i))."""
    lib = _load()
    target = _logits(target, dtype)
    B, g1, V = target.shape
    g = g1 - 1
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, g)
    u = np.ascontiguousarray(uniforms)
    if u.shape != (B, g + 1):
        raise ValueError("uniforms must be [B, gamma+1]")
    acc = np.empty(B, np.int32)
    out = np.empty((B, g + 1), np.int32)
    margin = np.empty(B, np.float64)
    ratios = np.empty((B, g), np.float64)
    fb = np.empty(B, np.int32)
    dist = np.empty((B, V), np.float64) if want_dist else None
    nt = default_threads() if threads is None else threads
    fn = lib.oracle_chain_pointmass_du if u.dtype == np.float64 else lib.oracle_chain_pointmass
    if u.dtype != np.float64:
        u = np.ascontiguousarray(u, dtype=np.float32)
    rc = fn(_ptr(target), _DT[dtype], _ptr(tok), _ptr(u), B, g, V, float(T), _ptr(acc), _ptr(out),
            _ptr(dist), _ptr(margin), _ptr(ratios), _ptr(fb), nt)
    if rc != 0:
        raise ValueError(f"oracle_chain_pointmass rejected its arguments (rc={rc})")
    return dict(accept_len=acc, out_tokens=out, margin=margin, ratios=ratios, fallback=fb,
                final_dist=dist)


def outcome_topk(logits, draft_tokens, T, ncache, dtype="f32", want_all=False) -> dict:
    """Outcome scores P(k, a) of a block from decoder rows [R, gamma+1, V] and
    the cache of the ncache most probable outcomes: k, a [R, ncache] (-1 in
    unused slots), p [R, ncache], hit [R] (the sum of the kept p; -1 for an
    invalid request) and, if asked, every score [R, gamma+1, V]."""
    lib = _load()
    logits = _logits(logits, dtype)
    R, g1, V = logits.shape
    g = g1 - 1
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(R, g)
    k = np.empty((R, ncache), np.int32)
    a = np.empty((R, ncache), np.int32)
    p = np.empty((R, ncache), np.float64)
    hit = np.empty(R, np.float64)
    allp = np.empty((R, g1, V), np.float64) if want_all else None
    rc = lib.oracle_outcome_topk(_ptr(logits), _DT[dtype], _ptr(tok), R, g, V, float(T),
                                 int(ncache), _ptr(k), _ptr(a), _ptr(p), _ptr(hit), _ptr(allp))
    if rc != 0:
        raise ValueError(f"oracle_outcome_topk rejected its arguments (rc={rc})")
    return dict(k=k, a=a, p=p, hit=hit, all_scores=allp)


def chain_alpha(target, draft, T, dtype="f32", threads=None) -> np.ndarray:
    """alpha[b, i] = sum_v min(p_i(v), q_i(v)), the acceptance probability at
    draft position i when the draft token is drawn from q_i."""
    lib = _load()
    target = _logits(target, dtype)
    draft = _logits(draft, dtype)
    B, g1, V = target.shape
    out = np.empty((B, g1 - 1), np.float64)
    nt = default_threads() if threads is None else threads
    rc = lib.oracle_chain_alpha(_ptr(target), _ptr(draft), _DT[dtype], B, g1 - 1, V, float(T),
                                _ptr(out), nt)
    if rc != 0:
        raise ValueError("oracle_chain_alpha rejected its arguments")
    return out


def tree_greedy(target, parents, tokens, dtype="bf16", threads=None) -> dict:
    """Greedy tree verification: deepest root path whose tokens all equal the
    target argmax after their parent, then the argmax after that path."""
    lib = _load()
    target = _logits(target, dtype)
    B, n, V = target.shape
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, n)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, n)
    acc = np.empty(B, np.int32)
    node = np.empty(B, np.int32)
    out = np.empty((B, n), np.int32)
    amax = np.empty((B, n), np.int32)
    nt = default_threads() if threads is None else threads
    rc = lib.oracle_tree_greedy(_ptr(target), _DT[dtype], _ptr(par), _ptr(tok), B, n, V,
                                _ptr(acc), _ptr(node), _ptr(out), _ptr(amax), nt)
    if rc != 0:
        raise ValueError("oracle_tree_greedy rejected its arguments")
    return dict(accept_len=acc, accept_node=node, out_tokens=out, amax=amax)




def tree_stochastic(target, draft, parents, tokens, uniforms, T, dtype="bf16",
                    want_dist=False) -> dict:
    """Stochastic tree verification: one Bernoulli test per node with
    probability min(1, p/q) from its parent's rows, the deepest node whose
    whole path passed wins, and the correction is drawn from p after it with
    u[:, 0].  float32 uniforms use the library's interface; float64 uniforms
    are taken as given (continuous-u enumeration in the tests).  Returns
    accept_len, accept_node [B], out_tokens [B, n], margin [B], alpha [B, n]
    (every node's test probability; NaN for the root) and, if asked,
    final_dist [B, V]."""
    lib = _load()
    target = _logits(target, dtype)
    draft = _logits(draft, dtype)
    B, n, V = target.shape
    if draft.shape != (B, n, V):
        raise ValueError("draft must have the target's shape [B, n, V]")
    par = np.ascontiguousarray(parents, dtype=np.int32)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    u = np.ascontiguousarray(uniforms)
    if u.shape != (B, n):
        raise ValueError("uniforms must be [B, n]")
    acc = np.empty(B, np.int32)
    node = np.empty(B, np.int32)
    out = np.empty((B, n), np.int32)
    margin = np.empty(B, np.float64)
    alpha = np.empty((B, n), np.float64)
    dist = np.empty((B, V), np.float64) if want_dist else None
    if u.dtype == np.float64:
        fn = lib.oracle_tree_stochastic_du
    else:
        fn = lib.oracle_tree_stochastic
        u = np.ascontiguousarray(u, dtype=np.float32)
    rc = fn(_ptr(target), _ptr(draft), _DT[dtype], _ptr(par), _ptr(tok), _ptr(u), B, n, V,
            float(T), _ptr(acc), _ptr(node), _ptr(out), _ptr(dist), _ptr(margin), _ptr(alpha))
    if rc != 0:
        raise ValueError(f"oracle_tree_stochastic rejected its arguments (rc={rc})")
    return dict(accept_len=acc, accept_node=node, out_tokens=out, margin=margin, alpha=alpha,
                final_dist=dist)

def tree_build(logits, T, W, N, budget, child_row=None, dtype="f32") -> dict:
    """Best-first construction of a draft tree from per-potential-node draft
    logits [R, M, V] ("JetSpec" reading notes, Algorithm 1 and Eq. 15).
    Returns parents, tokens, rows [R, budget] int32 (-1 past the end and for
    the root's parent and token), score [R, budget] float64 (natural log,
    -inf past the end), n [R] (-1 for an invalid request) and min_gap [R]
    (the smallest score gap behind an expansion decision)."""
    lib = _load()
    logits = _logits(logits, dtype)
    R, M, V = logits.shape
    cr = None
    if child_row is not None:
        cr = np.ascontiguousarray(child_row, dtype=np.int32)
        assert cr.shape == (M, W)
    par = np.empty((R, budget), np.int32)
    tok = np.empty((R, budget), np.int32)
    rows = np.empty((R, budget), np.int32)
    sc = np.empty((R, budget), np.float64)
    n = np.empty(R, np.int32)
    gap = np.empty(R, np.float64)
    rc = lib.oracle_tree_build(_ptr(logits), _DT[dtype], R, M, V, float(T), int(W), int(N),
                               int(budget), _ptr(cr), _ptr(par), _ptr(tok), _ptr(rows), _ptr(sc),
                               _ptr(n), _ptr(gap))
    if rc != 0:
        raise ValueError(f"oracle_tree_build rejected its arguments (rc={rc})")
    return dict(parents=par, tokens=tok, rows=rows, score=sc, n=n, min_gap=gap)

def tree_score(logits, parents, tokens, rows, n, T, dtype="f32") -> np.ndarray:
    """Scores [R, budget] of given trees under the draft rows [R, M, V]: the
    sum of ln q(token) along each node's path, each token in its parent's row
    ("JetSpec" reading notes, Eq. 15); -inf past the last node, NaN for a
    malformed tree."""
    lib = _load()
    logits = _logits(logits, dtype)
    R, M, V = logits.shape
    par = np.ascontiguousarray(parents, dtype=np.int32)
    budget = par.shape[1]
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    rw = np.ascontiguousarray(rows, dtype=np.int32)
    nn = np.ascontiguousarray(n, dtype=np.int32)
    assert par.shape == tok.shape == rw.shape == (R, budget) and nn.shape == (R,)
    sc = np.empty((R, budget), np.float64)
    rc = lib.oracle_tree_score(_ptr(logits), _DT[dtype], R, M, V, float(T), budget, _ptr(par),
                               _ptr(tok), _ptr(rw), _ptr(nn), _ptr(sc))
    if rc != 0:
        raise ValueError(f"oracle_tree_score rejected its arguments (rc={rc})")
    return sc


def cache_lookup(accept_len, out_tokens, cache_k, cache_a) -> np.ndarray:
    """The cache slot hit by each verified block ("JetSpec++", Section 4.2:
    the block drafted for outcome (k, a) is used when verification ends in
    (k, a)).  The verified outcome is k = accept_len[r], a = out_tokens[r][k];
    the result is the first slot c with (cache_k, cache_a)[r][c] = (k, a),
    else -1 (also for an invalid block, accept_len = -1)."""
    accept_len = np.asarray(accept_len)
    out_tokens = np.asarray(out_tokens)
    cache_k = np.asarray(cache_k)
    cache_a = np.asarray(cache_a)
    R, g1 = out_tokens.shape
    slot = np.full(R, -1, dtype=np.int32)
    for r in range(R):
        k = int(accept_len[r])
        if not 0 <= k < g1:
            continue
        a = int(out_tokens[r, k])
        for c in range(cache_k.shape[1]):
            if cache_k[r, c] == k and cache_a[r, c] == a:
                slot[r] = c
                break
    return slot
