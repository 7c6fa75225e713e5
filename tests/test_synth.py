"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 3, 1_000_000).astype(np.float32),
        rng.normal(0, 1e30, 1000).astype(np.float32),
        (rng.random(1000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                 np.float32),
    ])
    ours = synth.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    nan = synth.bf16_to_f32(synth.bf16_bits(np.array([np.nan], np.float32)))
    assert np.isnan(nan).all()


def test_bf16_widening_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_to_f32(bits)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (f == back) | (np.isnan(f) & np.isnan(back))
    assert same.all()


def test_deterministic_per_seed_and_thread_count():
    a = synth.chain_inputs(B=5, gamma=3, V=777, dtype="bf16", T=0.7, seed=42, threads=1)
    b = synth.chain_inputs(B=5, gamma=3, V=777, dtype="bf16", T=0.7, seed=42, threads=4)
    c = synth.chain_inputs(B=5, gamma=3, V=777, dtype="bf16", T=0.7, seed=43)
    for key in ("target", "draft", "draft_tokens", "uniforms"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["target"], c["target"])
    t1 = synth.tree_inputs(B=3, n=20, V=300, seed=1, threads=1)
    t2 = synth.tree_inputs(B=3, n=20, V=300, seed=1, threads=3)
    for key in ("target", "parents", "tokens"):
        assert np.array_equal(t1[key], t2[key])


def test_chain_distribution_moments():
    d = synth.chain_inputs(B=4, gamma=2, V=50_000, dtype="f32", T=1.0, target=("normal", 2.0),
                           noise=0.5, seed=1)
    t = d["target"].astype(np.float64)
    assert abs(t.mean()) < 0.02 and abs(t.std() - 2.0) < 0.02
    diff = d["draft"].astype(np.float64) - t[:, :2]
    assert abs(diff.std() - 0.5) < 0.01
    g = synth.chain_inputs(B=2, gamma=2, V=100_000, dtype="f32", target=("gumbel", 3.0),
                           seed=2)["target"].astype(np.float64) / 3.0
    assert abs(g.mean() - 0.5772156649) < 0.01 and abs(g.std() - np.pi / np.sqrt(6)) < 0.01
    u = d["uniforms"]
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()


def test_boost_and_draft_token_sampling():
    d = synth.config_inputs(3, seed=0, B=2, V=20_000, target=("normal", 0.1))
    z = synth.bf16_to_f32(d["target"]).astype(np.float64)
    assert ((z > 4.0).sum(axis=2) == 5).all()  # five distinct boosted ids per target row
    zd = synth.bf16_to_f32(d["draft"]).astype(np.float64)
    assert ((zd > 4.0).sum(axis=2) >= 4).all()  # the draft inherits them (plus N(0, 1) noise)
    d = synth.config_inputs(3, seed=0, B=2, V=20_000)
    tok = d["draft_tokens"]
    assert tok.dtype == np.int32 and ((tok >= 0) & (tok < 20_000)).all()


def test_gumbel_max_samples_softmax():
    """Frequency check of the draft-token sampler on a tiny vocabulary."""
    from scipy.special import softmax
    from scipy.stats import chisquare

    rng = np.random.default_rng(5)
    z = rng.normal(0, 1, 8).astype(np.float32)
    T = 0.7
    draws = []
    for s in range(300):
        g = synth._gumbel(np.random.default_rng(s), (200, 8))
        draws.append(np.argmax(z / np.float32(T) + g, axis=1))
    obs = np.bincount(np.concatenate(draws), minlength=8)
    p = softmax(z.astype(np.float64) / T)
    assert chisquare(obs, obs.sum() * p).pvalue > 1e-4


def test_tree_structure_and_planted_argmax():
    d = synth.tree_inputs(B=20, n=64, V=5000, max_depth=16, max_children=4, seed=3)
    par = d["parents"]
    assert (par[:, 0] == -1).all()
    for b in range(20):
        depth = np.zeros(64, int)
        nch = np.zeros(64, int)
        for j in range(1, 64):
            assert 0 <= par[b, j] < j
            depth[j] = depth[par[b, j]] + 1
            nch[par[b, j]] += 1
        assert depth.max() <= 16 and nch.max() <= 4
    z = synth.bf16_to_f32(d["target"])
    amax = np.argmax(z, axis=2)
    match = d["tokens"][:, 1:] == np.take_along_axis(amax, par[:, 1:], 1)
    assert 0.7 < match.mean() < 0.85
    assert abs(z.astype(np.float64).std() - 2.0) < 0.01


def test_tree_mask_ancestor_property():
    """Fig. 3 of the JetSpec notes: node v attends to u iff u is v or one of
    its ancestors; siblings' branches are invisible.  Check the ancestor
    relation implied by generated parent arrays."""
    d = synth.tree_inputs(B=5, n=30, V=100, seed=6)
    for par in d["parents"]:
        n = len(par)
        anc = np.zeros((n, n), bool)
        for v in range(n):
            u = v
            while u != -1:
                anc[v, u] = True
                u = par[u]
        assert anc[:, 0].all()  # every node sees the root
        for v in range(n):
            for u in range(n):
                if anc[v, u] and u != v:
                    assert not anc[u, v]  # antisymmetric
        # two children of one node never see each other
        for p in range(n):
            kids = np.nonzero(par == p)[0]
            for a in kids:
                for b in kids:
                    if a != b:
                        assert not anc[a, b]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_bytes(cfg):
    want = {1: 36_864, 2: 20_055_552, 3: 641_777_664, 4: 1_244_659_712, 5: 2_567_110_656}
    assert synth.config_bytes(cfg) == want[cfg]


def test_pointmass_inputs():
    a = synth.pointmass_inputs(6, 4, 500, "bf16", T=0.7, p_match=0.8, seed=5)
    b = synth.pointmass_inputs(6, 4, 500, "bf16", T=0.7, p_match=0.8, seed=5, threads=1)
    for k in ("target", "draft_tokens", "uniforms"):
        assert np.array_equal(a[k], b[k])
    # tokens are the target row's argmax about p_match of the time
    d = synth.pointmass_inputs(400, 4, 300, "f32", p_match=0.8, seed=6)
    amax = np.argmax(d["target"][:, :4], axis=2)
    rate = (d["draft_tokens"] == amax).mean()
    assert 0.76 < rate < 0.84
    assert synth.pointmass_config_bytes(3) == 64 * 17 * 151936 * 2


def test_treebuild_inputs():
    d = synth.treebuild_inputs(3, 21, 500, "bf16", logits=("gumbel", 2.0), seed=4)
    assert d["logits"].shape == (3, 21, 500) and d["logits"].dtype == np.uint16
    e = synth.treebuild_inputs(3, 21, 500, "bf16", logits=("gumbel", 2.0), seed=4, threads=1)
    assert np.array_equal(d["logits"], e["logits"])  # per-request streams: thread count free
    assert synth.complete_tree_rows(4, 4) == 85 and synth.complete_tree_rows(1, 5) == 5
    c = synth.TREEBUILD_CONFIG
    assert synth.treebuild_config_bytes() == (c["R"] * synth.complete_tree_rows(c["W"], c["N"])
                                             * c["V"] * 2)


def test_stree_inputs_structure_and_token_law():
    """Parents precede children within the caps; each node's token follows
    q at its parent (Gumbel-max): over many requests, the token equals the
    parent draft row's argmax about as often as the softmax predicts."""
    d = synth.stree_inputs(40, 12, 30, "f32", T=1.0, target=("normal", 1.0), noise=0.5,
                           max_depth=4, max_children=3, seed=5)
    par, tok = d["parents"], d["tokens"]
    assert (par[:, 0] == -1).all()
    hit, want = 0, 0.0
    for b in range(40):
        depth = np.zeros(12, int)
        for j in range(1, 12):
            assert 0 <= par[b, j] < j
            depth[j] = depth[par[b, j]] + 1
            q = np.exp(d["draft"][b, par[b, j]].astype(np.float64))
            q /= q.sum()
            want += q.max()
            hit += tok[b, j] == int(np.argmax(d["draft"][b, par[b, j]]))
        assert depth.max() <= 4 and np.bincount(par[b, 1:], minlength=12).max() <= 3
    n = 40 * 11
    assert abs(hit - want) < 5 * np.sqrt(want * (1 - want / n))
    assert ((d["uniforms"] >= 0) & (d["uniforms"] < 1)).all()
    assert synth.stree_config_bytes() == 2 * 64 * 64 * 151936 * 2
