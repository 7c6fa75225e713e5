"""The final draw's map from its uniform to a token, pinned against NumPy's
own inverse-transform sampler.

The pages fix the law of the final draw ("Speculative decoding verifies
draft tokens ...", section "Rejection uses a residual distribution"): the
residual max(0, p - q) renormalised after a rejection, p itself after a fully
accepted block, and p without the rejected token for a point-mass draft.  The
oracle turns the draw's uniform u into a token by walking the cumulative
weights in ascending token id and taking the first token whose cumulative
weight exceeds u times the total.  NumPy's Generator.choice(V, p=p) samples
the same way: it takes one Generator.random() value and returns the first
index whose normalised cumulative probability exceeds it.  So with u the
first random() of a seeded generator, the oracle must return the token that
choice() returns from a second generator of the same seed.  The weights
NumPy samples from are formed here, independently of the oracle, with
SciPy's softmax in fp64; a walk in any other order, an off-by-one at the
crossing or a wrong residual fails these tests."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def f32(x):
    return np.asarray(x, dtype=np.float32)


def clear_of_boundaries(p, u, eps=1e-12):
    """u is not within eps of a cumulative probability of p (where fp64
    rounding could send the two samplers to neighbouring tokens)."""
    c = np.cumsum(p)
    c /= c[-1]
    return bool(np.min(np.abs(c - u)) > eps)


def numpy_draw(p, seed):
    """The uniform NumPy's sampler uses, and its token."""
    u = np.random.default_rng(seed).random()
    tok = int(np.random.default_rng(seed).choice(len(p), p=p))
    return u, tok


V_CASES = [2, 7, 64, 1000]


@pytest.mark.parametrize("V", V_CASES)
def test_bonus_draw_map(V):
    """A fully accepted block (the draft equals the target, so every ratio
    is 1) draws from p_gamma."""
    checked = 0
    for s in range(60):
        rng = np.random.default_rng(9000 + 100 * V + s)
        tgt = f32(rng.normal(0, 2.0, (1, 2, V)))
        drf = tgt[:, :1].copy()
        x0 = int(rng.integers(0, V))
        p1 = softmax(tgt[0, 1].astype(np.float64))
        u1, ref = numpy_draw(p1, 77000 + s)
        if not clear_of_boundaries(p1, u1):
            continue
        r = oracle.chain(tgt, drf, np.array([[x0]]), np.array([[0.5, u1]]), 1.0)
        assert r["accept_len"][0] == 1
        assert r["out_tokens"][0, 1] == ref, (V, s)
        checked += 1
    assert checked >= 55


@pytest.mark.parametrize("V", V_CASES)
def test_residual_draw_map(V):
    """A rejection at the first position draws from max(0, p - q),
    renormalised."""
    checked = 0
    for s in range(60):
        rng = np.random.default_rng(9500 + 100 * V + s)
        tgt = f32(rng.normal(0, 2.0, (1, 2, V)))
        drf = f32(tgt[:, :1] + rng.normal(0, 1.0, (1, 1, V)))
        p0 = softmax(tgt[0, 0].astype(np.float64))
        q0 = softmax(drf[0, 0].astype(np.float64))
        over = np.flatnonzero(q0 > p0 * (1 + 1e-6))
        if len(over) == 0:
            continue
        x0 = int(over[rng.integers(0, len(over))])
        ratio = p0[x0] / q0[x0]
        res = np.maximum(p0 - q0, 0.0)
        res /= res.sum()
        u1, ref = numpy_draw(res, 78000 + s)
        if not clear_of_boundaries(res, u1):
            continue
        u0 = ratio + 0.5 * (1.0 - ratio)  # past the acceptance boundary: a rejection
        r = oracle.chain(tgt, drf, np.array([[x0]]), np.array([[u0, u1]]), 1.0)
        assert r["accept_len"][0] == 0
        assert r["out_tokens"][0, 0] == ref, (V, s)
        checked += 1
    assert checked >= 50


@pytest.mark.parametrize("V", V_CASES)
def test_pointmass_residual_draw_map(V):
    """A point-mass draft rejected at the first position draws from p
    without the rejected token, renormalised."""
    checked = 0
    for s in range(60):
        rng = np.random.default_rng(9900 + 100 * V + s)
        tgt = f32(rng.normal(0, 2.0, (1, 2, V)))
        p0 = softmax(tgt[0, 0].astype(np.float64))
        x0 = int(rng.integers(0, V))
        if p0[x0] > 1.0 - 1e-6:
            continue
        res = p0.copy()
        res[x0] = 0.0
        res /= res.sum()
        u1, ref = numpy_draw(res, 79000 + s)
        if not clear_of_boundaries(res, u1):
            continue
        u0 = p0[x0] + 0.5 * (1.0 - p0[x0])
        r = oracle.chain_pointmass(tgt, np.array([[x0]]), np.array([[u0, u1]]), 1.0)
        assert r["accept_len"][0] == 0
        assert r["out_tokens"][0, 0] == ref, (V, s)
        checked += 1
    assert checked >= 55
