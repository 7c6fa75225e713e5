"""Pins of the oracle's chain verification against what the pages and the
mathematics fix.  CPU only.

Each test drives the oracle as a black box (its uniforms in, (k, tokens) out)
and compares with a value the pages print, a closed form, or a law derived
independently here; a dropped term, a swapped p/q, a wrong comparison or an
off-by-one in the scan fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth
from enumerate_law import outcome_law

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def logp(p):
    """Logits whose softmax is p (float32 -> exact f64 inputs for the oracle)."""
    with np.errstate(divide="ignore"):
        return f32(np.log(np.asarray(p, dtype=np.float64)))


def onehot_logits(V, d):
    z = np.full(V, -np.inf, dtype=np.float32)
    z[d] = 0.0
    return z


def probs(z, T=1.0):
    return softmax(np.asarray(z, dtype=np.float64) / T)


# --------------------------------------------------------------------------
# Softmax (temperature softmax of each row)


def _bonus_dist(z_bonus, T):
    """final_dist of a block whose single test always passes (p = q), i.e. the
    bonus-row distribution p_gamma."""
    V = len(z_bonus)
    row0 = f32(np.linspace(-1, 1, V))
    tgt = np.stack([row0, f32(z_bonus)])[None]
    drf = row0[None, None]
    u = np.array([[0.5, 0.3]], dtype=np.float32)
    r = oracle.chain(tgt, drf, np.array([[0]]), u, T, want_dist=True)
    assert r["accept_len"][0] == 1
    return r["final_dist"][0]


@pytest.mark.parametrize("z1,z2,T", [(0.0, 0.0, 1.0), (1.5, -0.25, 1.0), (3.0, 2.0, 0.05),
                                     (-7.0, 4.0, 5.0), (10000.0, -10000.0, 1.0)])
def test_softmax_two_tokens_closed_form(z1, z2, T):
    dist = _bonus_dist([z1, z2], T)
    p1 = 1.0 / (1.0 + np.exp((np.float64(f32(z2)) - np.float64(f32(z1))) / T))
    assert abs(dist[0] - p1) < 1e-15
    assert abs(dist[1] - (1.0 - p1)) < 1e-15


def test_softmax_matches_library_softmax():
    rng = np.random.default_rng(5)
    for T in (0.3, 1.0, 2.5):
        z = f32(rng.normal(0, 3, 97))
        assert np.allclose(_bonus_dist(z, T), probs(z, T), rtol=0, atol=1e-14)


def test_masked_tokens_are_impossible():
    z = f32([1.0, -np.inf, 0.5, -np.inf])
    dist = _bonus_dist(z, 1.0)
    assert dist[1] == 0.0 and dist[3] == 0.0
    assert np.allclose(dist, probs(z), atol=1e-15)


# --------------------------------------------------------------------------
# Ratio test


def test_counterexample_two_thirds():
    """JetSpec++ Appendix F.3: q(d) = 0.9, p(d) = 0.6 commits d w.p. 2/3."""
    g = gold("counterexample_f3.json")
    tgt = np.stack([logp([g["p_d"], 1 - g["p_d"]]), logp([0.5, 0.5])])
    drf = logp([g["q_d"], 1 - g["q_d"]])[None]
    law, t = outcome_law(tgt, drf, [0])
    assert abs(t[0] - g["commit_probability"]) < 1e-7  # float32 logits of 0.6/0.9
    # committing d means accepting it (k = 1); the residual never emits d
    p_commit = sum(m for (k, v), m in law.items() if k == 1)
    exact = np.exp(np.float64(tgt[0, 0]) - np.log(np.exp(np.float64(tgt[0])).sum())) / \
        np.exp(np.float64(drf[0, 0]) - np.log(np.exp(np.float64(drf[0])).sum()))
    assert abs(p_commit - exact) < 1e-15
    assert all(v != 0 for (k, v) in law if k == 0)


def test_ratio_and_margin_outputs():
    tgt = np.stack([logp([0.2, 0.8]), logp([0.5, 0.5])])[None]
    drf = logp([0.4, 0.6])[None, None]
    for u, k in ((0.49, 1), (0.51, 0)):
        r = oracle.chain(tgt, drf, np.array([[0]]), np.array([[u, 0.5]], np.float32), 1.0)
        assert abs(r["ratios"][0, 0] - 0.5) < 1e-7
        assert r["accept_len"][0] == k
        assert r["margin"][0] <= abs(np.float32(u) - r["ratios"][0, 0]) + 1e-15
    # p(x) = 0.8 > q(x) = 0.6: the ratio is capped at exactly 1 and the test
    # sits 1 - u away from its boundary
    r = oracle.chain(tgt, drf, np.array([[1]]), np.array([[0.25, 0.5]], np.float32), 1.0)
    assert r["ratios"][0, 0] == 1.0 and r["accept_len"][0] == 1
    assert r["margin"][0] <= 0.75 + 1e-15


def test_acceptance_probability_is_sum_of_min():
    """P(test passes) = sum_x q(x) min(1, p(x)/q(x)) = sum_v min(p(v), q(v))."""
    rng = np.random.default_rng(11)
    V = 6
    for T in (0.7, 1.0, 1.8):
        zp = f32(rng.normal(0, 1.5, (2, V)))
        zq = f32(zp[:1] + rng.normal(0, 1.0, (1, V)))
        p, q = probs(zp[0], T), probs(zq[0], T)
        total = 0.0
        for x in range(V):
            _, t = outcome_law(zp, zq, [x], T=T)
            total += q[x] * t[0]
        assert abs(total - np.minimum(p, q).sum()) < 1e-14
        alpha = oracle.chain_alpha(zp[None], zq[None], T)[0, 0]
        assert abs(alpha - np.minimum(p, q).sum()) < 1e-14


# --------------------------------------------------------------------------
# Residual and bonus


def test_worked_example_024():
    """JetSpec++ Appendix F.1: P(end at (1, b)) = 0.8 * 0.5 * 0.6 = 0.24."""
    g = gold("worked_example_f1.json")
    # tokens: 0 = d1 = d2, 1 = b, 2 = another token
    p1 = [g["p1"]["d1"], g["p1"]["other"] / 2, g["p1"]["other"] / 2]
    p2 = [g["p2"]["d2"], g["p2"]["b"], g["p2"]["rest"]]
    tgt = np.stack([logp(p1), logp(p2), logp([0.2, 0.3, 0.5])])
    drf = np.stack([onehot_logits(3, 0), onehot_logits(3, 0)])
    law, t = outcome_law(tgt, drf, [0, 0])
    assert abs(t[0] - g["p_accept_d1"]) < 1e-7
    assert abs((1 - t[1]) - g["p_reject_d2"]) < 1e-7
    assert abs(law[(1, 1)] - g["p_end_at_1_b"]) < 1e-7
    # The same value from the exactly decoded float32 logits, to 1e-15.
    P1, P2 = probs(tgt[0]), probs(tgt[1])
    assert abs(law[(1, 1)] - P1[0] * P2[1]) < 1e-15
    # the rejected draft token is never emitted by the residual
    assert (1, 0) not in law


@pytest.mark.parametrize("seed", range(4))
def test_proposition1_point_mass_law(seed):
    """JetSpec++ Proposition 1: with q_i = delta_{d_i}, the outcome law is
    P(k, a) = prod_{j<k} p_j(d_j) * p_k(a) for a != d_k (k < gamma), and
    P(gamma, a) = prod_j p_j(d_j) * p_gamma(a)."""
    rng = np.random.default_rng(100 + seed)
    V, g = 4, 3
    tgt = f32(rng.normal(0, 1.2, (g + 1, V)))
    d = rng.integers(0, V, g)
    drf = np.stack([onehot_logits(V, x) for x in d])
    law, _ = outcome_law(tgt, drf, d)
    P = [probs(tgt[j]) for j in range(g + 1)]
    want = {}
    run = 1.0
    for k in range(g + 1):
        for a in range(V):
            if k < g and a == d[k]:
                continue
            want[(k, a)] = run * P[k][a]
        if k < g:
            run *= P[k][d[k]]
    keys = set(want) | set(law)
    for key in keys:
        assert abs(law.get(key, 0.0) - want.get(key, 0.0)) < 1e-14, key
    assert abs(sum(law.values()) - 1.0) < 1e-14


@pytest.mark.parametrize("T", [0.6, 1.0])
def test_committed_token_law_equals_target(T):
    """Lossless output ("Speculative decoding verifies draft tokens ...",
    section "Rejection uses a residual distribution"): over successive
    rounds, the law of the first L committed tokens equals prod p(t_j | t_<j).

    Toy model: target and draft logits are tables indexed by the whole prefix;
    all drafts (weighted by their draft probability) and all outcomes of the
    oracle (weighted by their exact probability) are enumerated."""
    V, g, L = 3, 2, 3

    def table(which, prefix):
        rng = np.random.default_rng([which, len(prefix)] + list(prefix))
        return f32(rng.normal(0, 1.3, V))

    def tgt_logits(prefix):
        return table(1, prefix)

    def drf_logits(prefix):
        return f32(tgt_logits(prefix) + table(2, prefix))

    law = {}

    def expand(prefix, prob):
        if len(prefix) >= L:
            key = tuple(prefix[:L])
            law[key] = law.get(key, 0.0) + prob
            return
        for draft in itertools.product(range(V), repeat=g):
            qd = 1.0
            for i in range(g):
                qd *= probs(drf_logits(prefix + list(draft[:i])), T)[draft[i]]
            tgt = np.stack([tgt_logits(prefix + list(draft[:i])) for i in range(g + 1)])
            drf = np.stack([drf_logits(prefix + list(draft[:i])) for i in range(g)])
            outcomes, _ = outcome_law(tgt, drf, np.array(draft), T=T)
            for (k, tok), m in outcomes.items():
                expand(prefix + list(draft[:k]) + [tok], prob * qd * m)

    expand([], 1.0)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    for seq in itertools.product(range(V), repeat=L):
        want = 1.0
        for j in range(L):
            want *= probs(tgt_logits(list(seq[:j])), T)[seq[j]]
        assert abs(law.get(seq, 0.0) - want) < 1e-12, seq


# --------------------------------------------------------------------------
# Accept length


def _iid_rows(alpha):
    """Per position p = (1/2, 1/2), q = (3/2 - alpha, alpha - 1/2), so that
    sum_v min(p, q) = alpha for alpha in [1/2, 1)."""
    return logp([0.5, 0.5]), logp([1.5 - alpha, alpha - 0.5])


def test_expected_tokens_closed_form_enumerated():
    """JetSpec reading notes Eq. 2: E[k + 1] = (1 - alpha^(N+1)) / (1 - alpha)."""
    case = gold("expected_tokens_eq2.json")["cases"][0]
    alpha, N = case["alpha"], case["N"]
    zp, zq = _iid_rows(alpha)
    q = probs(zq)
    tgt = np.stack([zp] * (N + 1))
    drf = np.stack([zq] * N)
    exact_alpha = np.minimum(probs(zp), q).sum()
    expect = 0.0
    for draft in itertools.product(range(2), repeat=N):
        w = np.prod([q[x] for x in draft])
        law, _ = outcome_law(tgt, drf, np.array(draft))
        expect += w * sum((k + 1) * m for (k, _tok), m in law.items())
    closed = (1 - exact_alpha ** (N + 1)) / (1 - exact_alpha)
    assert abs(expect - closed) < 1e-12
    assert abs(closed - case["expected"]) < 1e-6  # float32 rounding of q


def test_expected_tokens_closed_form_monte_carlo():
    case = gold("expected_tokens_eq2.json")["cases"][1]
    alpha, N = case["alpha"], case["N"]
    zp, zq = _iid_rows(alpha)
    a = np.minimum(probs(zp), probs(zq)).sum()
    B = 200_000
    rng = np.random.default_rng(7)
    tgt = np.broadcast_to(np.stack([zp] * (N + 1)), (B, N + 1, 2)).copy()
    drf = np.broadcast_to(np.stack([zq] * N), (B, N, 2)).copy()
    d = (rng.random((B, N)) < probs(zq)[1]).astype(np.int32)
    u = rng.random((B, N + 1), dtype=np.float32)
    r = oracle.chain(tgt, drf, d, u, 1.0)
    mean = (r["accept_len"] + 1).mean()
    closed = (1 - a ** (N + 1)) / (1 - a)
    ks = np.arange(N + 1)
    pk = np.where(ks < N, a ** ks * (1 - a), a ** N)
    sd = np.sqrt(((ks + 1) ** 2 * pk).sum() - closed ** 2)
    assert abs(mean - closed) < 4 * sd / np.sqrt(B)
    assert abs(closed - case["expected"]) < 1e-6


def test_acceptance_frequency_monte_carlo():
    """Empirical pass rate at every position against sum_v min(p, q)."""
    d = synth.chain_inputs(B=4000, gamma=3, V=40, dtype="f32", T=0.8,
                           target=("normal", 1.5), noise=0.6, seed=3)
    r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"])
    alpha = oracle.chain_alpha(d["target"], d["draft"], d["T"])
    k = r["accept_len"]
    for i in range(3):
        reached = k >= i
        passed = k[reached] > i
        a = alpha[reached, i]
        sd = np.sqrt((a * (1 - a)).sum())
        assert abs(passed.sum() - a.sum()) < 4.5 * sd, i


def test_emitted_first_token_follows_target_chi2():
    """With gamma = 1 the first committed token (accepted draft or residual
    draw) must follow p_0; chi-square over 10^5 draws on V = 16."""
    from scipy.stats import chisquare

    rng = np.random.default_rng(21)
    V, B, T = 16, 100_000, 1.0
    zp = f32(rng.normal(0, 1.0, (2, V)))
    zq = f32(zp[0] + rng.normal(0, 0.8, V))
    q = probs(zq, T)
    d = rng.choice(V, size=B, p=q).astype(np.int32)[:, None]
    tgt = np.broadcast_to(zp, (B, 2, V)).copy()
    drf = np.broadcast_to(zq[None], (B, 1, V)).copy()
    u = rng.random((B, 2), dtype=np.float32)
    r = oracle.chain(tgt, drf, d, u, T)
    first = r["out_tokens"][:, 0]
    obs = np.bincount(first, minlength=V)
    p = probs(zp[0], T)
    stat, pval = chisquare(obs, B * p)
    assert pval > 1e-4, (stat, pval)


# --------------------------------------------------------------------------
# Edge cases and invalid blocks


def test_all_accept_when_draft_equals_target():
    d = synth.chain_inputs(B=50, gamma=5, V=33, dtype="bf16", T=0.9, seed=8)
    drf = d["target"][:, :5].copy()
    r = oracle.chain(d["target"], drf, d["draft_tokens"], d["uniforms"], 0.9, dtype="bf16")
    assert (r["accept_len"] == 5).all()
    assert (r["out_tokens"][:, :5] == d["draft_tokens"]).all()


def test_token_is_always_in_support():
    d = synth.chain_inputs(B=300, gamma=4, V=50, dtype="f32", T=1.3, seed=9)
    r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], 1.3,
                     want_dist=True)
    for b in range(300):
        k = r["accept_len"][b]
        tok = r["out_tokens"][b, k]
        assert r["final_dist"][b, tok] > 0.0
        assert abs(r["final_dist"][b].sum() - 1.0) < 1e-12
        assert (r["out_tokens"][b, k + 1:] == -1).all()


def test_residual_excludes_overweighted_tokens():
    d = synth.chain_inputs(B=200, gamma=2, V=30, dtype="f32", T=1.0, seed=10)
    r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], 1.0,
                     want_dist=True)
    for b in np.nonzero(r["accept_len"] < 2)[0]:
        k = r["accept_len"][b]
        p = probs(d["target"][b, k])
        q = probs(d["draft"][b, k])
        w = np.maximum(p - q, 0)
        assert np.allclose(r["final_dist"][b], w / w.sum(), atol=1e-13)


@pytest.mark.parametrize("kind", ["nan", "posinf", "allneginf", "token_hi", "token_neg"])
def test_invalid_block_is_flagged_alone(kind):
    d = synth.chain_inputs(B=3, gamma=3, V=20, dtype="f32", T=1.0, seed=12)
    tgt, drf, tok = d["target"].copy(), d["draft"].copy(), d["draft_tokens"].copy()
    if kind == "nan":
        drf[1, 2, 5] = np.nan
    elif kind == "posinf":
        tgt[1, 3, 0] = np.inf
    elif kind == "allneginf":
        tgt[1, 0, :] = -np.inf
    elif kind == "token_hi":
        tok[1, 2] = 20
    else:
        tok[1, 0] = -1
    ref = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], 1.0)
    r = oracle.chain(tgt, drf, tok, d["uniforms"], 1.0)
    assert r["accept_len"][1] == -1 and (r["out_tokens"][1] == -1).all()
    for b in (0, 2):
        assert r["accept_len"][b] == ref["accept_len"][b]
        assert (r["out_tokens"][b] == ref["out_tokens"][b]).all()


@pytest.mark.parametrize("T,shift", [(1e-6, 300.0), (1.0, 3.0e8), (1e-6, -5.0e4)])
def test_huge_scaled_logits_follow_the_definition(T, shift):
    """Rows whose logits divided by T are enormous are ordinary inputs for the
    rule: p = softmax(z / T) in double precision.  The ratios and the draw
    distribution must equal scipy's log_softmax / softmax of the same
    decoded values (an independent library), and the outcome must be the one
    those probabilities give."""
    from scipy.special import log_softmax, softmax

    rng = np.random.default_rng(71)
    g, V = 3, 50
    tgt = f32(shift + rng.normal(0, 2e-4 if abs(shift) < 1e3 else 64.0, (g + 1, V)))
    drf = f32(tgt[:g] + f32(rng.normal(0, 1e-4 if abs(shift) < 1e3 else 64.0, (g, V))))
    tok = np.array([int(np.argmax(tgt[0])), int(np.argmax(drf[1])), 7], np.int32)
    u = np.array([[0.3, 0.6, 0.9, 0.45]], np.float32)
    r = oracle.chain(tgt[None], drf[None], tok[None], u, T, want_dist=True)
    lp = log_softmax(tgt.astype(np.float64) / T, axis=1)
    lq = log_softmax(drf.astype(np.float64) / T, axis=1)
    with np.errstate(over="ignore"):
        want_r = [min(1.0, float(np.exp(lp[i, tok[i]] - lq[i, tok[i]]))) for i in range(g)]
    assert np.allclose(r["ratios"][0], want_r, rtol=1e-12, atol=1e-300)
    k = next((i for i in range(g) if not u[0, i] < want_r[i]), g)
    assert r["accept_len"][0] == k
    if k < g:
        w = np.maximum(softmax(tgt[k].astype(np.float64) / T) - softmax(drf[k].astype(np.float64) / T), 0)
    else:
        w = softmax(tgt[g].astype(np.float64) / T)
    assert np.allclose(r["final_dist"][0], w / w.sum(), atol=1e-12)


def test_masked_draft_token_rules():
    """q(x) = 0 < p(x) accepts (r = 1); p(x) = 0 rejects (r = 0)."""
    ninf = -np.inf
    tgt = f32([[0.0, 1.0, ninf], [0.0, 0.0, 0.0]])
    drf = f32([[0.0, ninf, 0.0]])
    u = np.array([[0.999, 0.5]], np.float32)
    r = oracle.chain(tgt[None], drf[None], np.array([[1]]), u, 1.0)
    assert r["ratios"][0, 0] == 1.0 and r["accept_len"][0] == 1
    u = np.array([[0.0, 0.5]], np.float32)
    r = oracle.chain(tgt[None], drf[None], np.array([[2]]), u, 1.0, want_dist=True)
    assert r["ratios"][0, 0] == 0.0 and r["accept_len"][0] == 0
    # residual max(0, p - q) puts no mass on token 2 (p = 0) and keeps token 1
    assert r["final_dist"][0, 2] == 0.0 and r["final_dist"][0, 1] > 0.0


def test_uniform_zero_and_top_of_range():
    """u = 0 passes any test with r > 0; the largest float32 below 1 fails
    every test with r < 1 and picks the last token of positive mass."""
    d = synth.chain_inputs(B=20, gamma=3, V=25, dtype="f32", T=1.0, seed=13)
    u0 = np.zeros_like(d["uniforms"])
    r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], u0, 1.0)
    assert (r["accept_len"] == 3).all()
    assert (r["out_tokens"][:, 3] == 0).all()  # first token of positive mass
    u1 = np.full_like(d["uniforms"], np.nextafter(np.float32(1), np.float32(0)))
    r = oracle.chain(d["target"], d["draft"], d["draft_tokens"], u1, 1.0)
    assert (r["ratios"][:, 0] < 1).sum() > 0
    for b in range(20):
        if r["ratios"][b, 0] < 1:
            assert r["accept_len"][b] == 0
