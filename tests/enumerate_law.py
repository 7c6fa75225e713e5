"""Exact law of the oracle's chain decision, found by treating the oracle as a
black box of its uniforms.

Each decision of a chain block is a monotone step function of one uniform: the
test at position i accepts for u_i below some threshold, and the final draw's
token is non-decreasing in u_gamma.  Bisection in double precision (60 halvings
per boundary, all boundaries of a block bisected together in one batched oracle
call) recovers every boundary to about 1e-18, so the probability of each
outcome (k, token) follows exactly from interval lengths, without reading the
oracle's internals.
"""
from __future__ import annotations

import numpy as np

import oracle

STEPS = 60
U_REJECT = float(np.nextafter(1.0, 0.0))  # largest double below 1


def _chain_runner(tgt, drf, tok, U, T, dtype):
    return oracle.chain(tgt, drf, tok, U, T, dtype=dtype, threads=1)


def _pointmass_runner(tgt, drf, tok, U, T, dtype):
    return oracle.chain_pointmass(tgt, tok, U, T, dtype=dtype, threads=1)


RUNNERS = {"chain": _chain_runner, "pointmass": _pointmass_runner}


def _run(target, draft, tokens, U, T, dtype, runner=_chain_runner):
    B = U.shape[0]
    tgt = np.broadcast_to(target, (B,) + target.shape).copy()
    drf = np.broadcast_to(draft, (B,) + draft.shape).copy()
    tok = np.broadcast_to(tokens, (B,) + tokens.shape).copy()
    return runner(tgt, drf, tok, U, T, dtype)


def outcome_law(target, draft, tokens, T=1.0, dtype="f32", rule="chain"):
    """Return {(k, token): probability} for one block.

    target [gamma+1, V], draft [gamma, V] (stored dtype; ignored by the
    point-mass rule), tokens [gamma]; rule "chain" (ratio test against the
    draft distribution) or "pointmass" (the draft proposes each token with
    certainty).
    """
    runner = RUNNERS[rule]
    target = np.asarray(target)
    draft = np.asarray(draft)
    tokens = np.asarray(tokens, dtype=np.int32)
    g = draft.shape[0]
    V = target.shape[1]

    # Acceptance thresholds t_i = sup{u_i : test i passes}, earlier tests forced
    # to pass with u = 0 (which passes whenever the threshold is positive).
    lo = np.zeros(g)
    hi = np.ones(g)
    U0 = np.zeros((g, g + 1))
    U0[np.arange(g), np.arange(g)] = 0.0
    first = _run(target, draft, tokens, U0, T, dtype, runner)["accept_len"]
    passes0 = first > np.arange(g)
    for _ in range(STEPS):
        mid = 0.5 * (lo + hi)
        U = np.zeros((g, g + 1))
        U[np.arange(g), np.arange(g)] = mid
        acc = _run(target, draft, tokens, U, T, dtype, runner)["accept_len"]
        ok = acc > np.arange(g)
        lo = np.where(ok, mid, lo)
        hi = np.where(ok, hi, mid)
    t = np.where(passes0, hi, 0.0)
    # every earlier test must be able to pass for a later one to be reached
    pk = np.zeros(g + 1)
    run = 1.0
    for i in range(g):
        pk[i] = run * (1.0 - t[i])
        run *= t[i]
    pk[g] = run

    # Token boundaries F_k(v) = sup{u : token(u) <= v} for every reachable k.
    ks = [k for k in range(g + 1) if pk[k] > 0.0]
    pairs = [(k, v) for k in ks for v in range(V)]
    n = len(pairs)
    base = np.zeros((n, g + 1))
    for r, (k, v) in enumerate(pairs):
        if k < g:
            base[r, k] = U_REJECT
    kk = np.array([p[0] for p in pairs])
    vv = np.array([p[1] for p in pairs])

    def token_at(u):
        U = base.copy()
        U[:, g] = u
        res = _run(target, draft, tokens, U, T, dtype, runner)
        assert np.array_equal(res["accept_len"], kk), "forced outcome k not reached"
        return res["out_tokens"][np.arange(n), kk]

    at0 = token_at(np.zeros(n))
    lo = np.zeros(n)
    hi = np.ones(n)
    for _ in range(STEPS):
        mid = 0.5 * (lo + hi)
        le = token_at(mid) <= vv
        lo = np.where(le, mid, lo)
        hi = np.where(le, hi, mid)
    F = np.where(at0 <= vv, hi, 0.0)
    law = {}
    for k in ks:
        Fk = F[kk == k]
        prev = 0.0
        for v in range(V):
            m = Fk[v] - prev
            prev = Fk[v]
            if m > 0.0:
                law[(k, v)] = pk[k] * m
    return law, t
