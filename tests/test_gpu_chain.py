"""GPU parity of spec_verify_chain against the fp64 oracle (needs an MI355X).

Every case draws seeded inputs, runs the HIP library through its C ABI and
the oracle on the same inputs, and compares with the rule in gpu_util: exact
accept lengths and tokens outside the 1e-6 boundary band, final_dist to 1e-5.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_chain, gpu_chain, require_gpu, to_dev, to_dev_logits

pytestmark = pytest.mark.gpu


def run_case(d, label, want_dist=True):
    print(f"[case] {label} B={d['B']} gamma={d['gamma']} V={d['V']} {d['dtype']} T={d['T']}",
          flush=True)
    g = gpu_chain(d, want_dist=want_dist)
    o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                     dtype=d["dtype"], want_dist=want_dist)
    n, near = compare_chain(g, o, label, d=d)
    print(f"[case] {label}: compared {n} blocks, {near} inside the boundary band", flush=True)
    return g, o


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


SHAPES = [(3, 1, 1), (5, 2, 7), (4, 31, 1000), (2, 3, 5003), (1, 16, 151937), (7, 4, 4096),
          (2, 255, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}g{g}V{v}" for b, g, v in SHAPES])
def test_shapes_and_ragged_tails(shape, dtype):
    B, g, V = shape
    for seed in range(3):
        d = synth.chain_inputs(B, g, V, dtype, T=0.9, target=("normal", 2.0), noise=0.6,
                               seed=1000 + seed)
        run_case(d, f"shape{shape}-{dtype}-s{seed}")


# Batches large enough that each final-draw workgroup streams a run of
# several tiles: a ratio-test chain's runs are capped at four tiles, so these
# give runs of 3 and 4 (the point-mass tests cover runs of up to 33), a
# ragged last run and tile, and vocabularies whose rows are not 16-byte
# aligned (mixed aligned and unaligned rows in one launch).
LONG_SHAPES = [(256, 2, 40000, "bf16"), (512, 1, 65541, "bf16"), (300, 2, 20000, "f32"),
               (300, 2, 20003, "f32"), (200, 3, 30000, "bf16")]


@pytest.mark.parametrize("shape", LONG_SHAPES, ids=[f"B{b}g{g}V{v}{t}" for b, g, v, t in LONG_SHAPES])
def test_long_chunk_runs(shape):
    B, g, V, dtype = shape
    d = synth.chain_inputs(B, g, V, dtype, T=0.8, target=("normal", 2.0), noise=0.6, seed=4100 + g)
    run_case(d, f"long{shape}")


# Seeded rounds at full size: 200 each of configs 1 and 2, 20 each of
# configs 3 and 5 (final_dist compared on every one), split into chunks so
# that each test stays well under a minute.
FULL_SIZE = ([(1, range(0, 200))] + [(2, range(i, i + 50)) for i in range(0, 200, 50)] +
             [(3, range(i, i + 5)) for i in range(0, 20, 5)] +
             [(5, range(i, i + 2)) for i in range(0, 20, 2)])


@pytest.mark.parametrize("cfg,seeds", FULL_SIZE,
                         ids=[f"config{c}-s{r.start}-{r.stop - 1}" for c, r in FULL_SIZE])
def test_configs_full_size(cfg, seeds):
    for s in seeds:
        d = synth.config_inputs(cfg, seed=1000 * cfg + s)
        run_case(d, f"config{cfg}-s{s}", want_dist=True)


# Per-position acceptance at full size: with every draft token drawn afresh
# from q_i, the test at position i, once reached, passes with probability
# alpha_i = sum_v min(p_i(v), q_i(v)) ("Speculative decoding verifies draft
# tokens ...", section "Rejection uses a residual distribution"; the
# oracle's chain_alpha).  Reaching position i depends only on earlier
# positions, so over all blocks and redraws the pass count at each position
# is a sum of independent Bernoulli(alpha) terms: z-test per position and
# pooled.  (logit seeds, redraws per seed) per configuration:
ACCEPT = {1: (20, 100), 2: (4, 150), 3: (1, 24), 5: (1, 8)}


@pytest.mark.parametrize("cfg", sorted(ACCEPT))
def test_acceptance_rate_matches_sum_min_full_size(cfg):
    torch, sv = require_gpu()
    nseed, nredraw = ACCEPT[cfg]
    g = synth.CONFIGS[cfg]["gamma"]
    passed = np.zeros(g)
    expect = np.zeros(g)
    var = np.zeros(g)
    for si in range(nseed):
        d = synth.config_inputs(cfg, seed=50000 + 1000 * cfg + si)
        print(f"[case] acceptance config{cfg} logits seed {si}: {nredraw} redraws", flush=True)
        alpha = oracle.chain_alpha(d["target"], d["draft"], d["T"], dtype=d["dtype"])
        tgt = to_dev_logits(d["target"], d["dtype"])
        drf = to_dev_logits(d["draft"], d["dtype"])
        for r in range(nredraw):
            tok, uni = synth.redraw_chain_tokens(d, seed=7 + 1000 * si + r)
            acc, _, _ = sv.spec_verify_chain(tgt, drf, to_dev(tok, np.int32),
                                             to_dev(uni, np.float32), d["T"])
            k = acc.cpu().numpy()
            assert (k >= 0).all()
            for i in range(g):
                reached = k >= i
                passed[i] += (k[reached] > i).sum()
                a = alpha[reached, i]
                expect[i] += a.sum()
                var[i] += (a * (1.0 - a)).sum()
    ok = var > 0
    z = (passed[ok] - expect[ok]) / np.sqrt(var[ok])
    zpool = (passed.sum() - expect.sum()) / np.sqrt(var.sum())
    print(f"[case] acceptance config{cfg}: per-position z {np.round(z, 2).tolist()}, pooled "
          f"{zpool:.2f}", flush=True)
    assert np.abs(z).max() < 4.5 and abs(zpool) < 4.5


def test_config3_more_uniforms():
    """Same logits, fresh uniforms: many more decisions at full size."""
    d = synth.config_inputs(3, seed=3001)
    rng = np.random.default_rng(5)
    for r in range(4):
        d["uniforms"] = rng.random(d["uniforms"].shape, dtype=np.float32)
        run_case(d, f"config3-u{r}", want_dist=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_accept_bonus_path(dtype):
    d = synth.chain_inputs(16, 5, 3000, dtype, T=0.8, seed=7)
    d["draft"] = d["target"][:, :5].copy()
    g, o = run_case(d, f"all-accept-{dtype}")
    assert (g["accept_len"] == 5).all()


def test_point_mass_drafts():
    """One-hot draft logits (-inf elsewhere): q = delta_d, the exact-match rule
    of JetSpec++ Appendix F.3 expressed through the ratio test."""
    d = synth.chain_inputs(32, 4, 2000, "f32", T=1.0, seed=8)
    drf = np.full_like(d["draft"], -np.inf)
    for b in range(32):
        for i in range(4):
            drf[b, i, d["draft_tokens"][b, i]] = 0.0
    d["draft"] = drf
    run_case(d, "point-mass")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masked_tokens(dtype):
    d = synth.chain_inputs(24, 6, 4099, dtype, T=1.1, seed=9)
    rng = np.random.default_rng(9)
    ninf = np.float32(-np.inf) if dtype == "f32" else np.uint16(0xFF80)
    for key in ("target", "draft"):
        arr = d[key]
        mask = rng.random(arr.shape) < 0.3
        arr[mask] = ninf
    # keep every draft token possible under q so the inputs stay meaningful
    for b in range(24):
        for i in range(6):
            x = d["draft_tokens"][b, i]
            d["draft"][b, i, x] = 0 if dtype == "bf16" else np.float32(0.0)
    run_case(d, f"masked-{dtype}")


@pytest.mark.parametrize("dtype,offset", [("f32", 1000.5), ("f32", -250.0), ("bf16", 37.25)])
def test_draft_logit_offset(dtype, offset):
    """Softmax ignores a constant shift of a row's logits, so draft logits that
    sit at an offset from the target's (as a different model's would) must
    still match the oracle; a close draft (small noise, acceptance near 1)
    makes the residual small and the test sensitive to cancellation."""
    d = synth.chain_inputs(48, 8, 30000, dtype, T=0.8, noise=0.15, seed=17)
    if dtype == "f32":
        d["draft"] = (d["draft"] + np.float32(offset)).astype(np.float32)
    else:
        shifted = synth.bf16_to_f32(d["draft"]) + np.float32(offset)
        d["draft"] = synth.bf16_bits(shifted)
    run_case(d, f"offset{offset}-{dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_near_identical_draft(dtype):
    """Draft logits within 0.03 of the target's: acceptance near 1, so after a
    rejection the residual max(0, p - q) holds a tiny share of the mass and
    every weight is a difference of nearly equal probabilities.  Uniforms are
    pushed toward 1 so that rejections (and residual draws) do happen."""
    d = synth.chain_inputs(64, 6, 20000, dtype, T=1.0, noise=0.03, seed=18)
    rng = np.random.default_rng(18)
    d["uniforms"] = (1.0 - 0.02 * rng.random(d["uniforms"].shape)).astype(np.float32)
    d["uniforms"][:, -1] = rng.random(64, dtype=np.float32)
    g, o = run_case(d, f"near-identical-{dtype}")
    assert (o["accept_len"] < 6).sum() >= 10  # the residual path is exercised


@pytest.mark.parametrize("dtype,noise,ueps", [("bf16", 0.1, 1e-3), ("bf16", 0.3, 1e-3),
                                              ("f32", 0.02, 1e-3), ("f32", 0.01, 1e-4)])
def test_small_residual_mass(dtype, noise, ueps):
    """Peaked rows at the full vocabulary with drafts close to the target, so
    that a rejection leaves a residual of small mass W (2e-5 to 5e-2 here):
    the regime where an error in the rows' log-normalisers is amplified by
    about 1/W in the draw.  Uniforms within ueps of 1 force rejections; the
    draw and final_dist must still match the oracle (1e-6 band, 1e-5
    absolute)."""
    d = synth.chain_inputs(24, 4, 151936, dtype, T=0.6, target=("gumbel", 4.0), noise=noise,
                           seed=19)
    rng = np.random.default_rng(19)
    d["uniforms"][:, :4] = (1.0 - ueps * rng.random((24, 4))).astype(np.float32)
    g, o = run_case(d, f"small-W-{dtype}-{noise}-{ueps}")
    assert (o["accept_len"] < 4).sum() >= 8  # residual draws happen


@pytest.mark.parametrize("T", [0.05, 5.0])
def test_temperature_extremes(T):
    d = synth.chain_inputs(16, 8, 10000, "bf16", T=T, target=("normal", 2.0), noise=0.3, seed=10)
    run_case(d, f"T{T}")


def test_large_logits():
    d = synth.chain_inputs(8, 4, 3000, "f32", T=1.0, seed=11)
    rng = np.random.default_rng(11)
    d["target"] = np.where(rng.random(d["target"].shape) < 0.5, 1e4, -1e4).astype(np.float32)
    d["draft"] = d["target"][:, :4] + rng.normal(0, 0.5, d["draft"].shape).astype(np.float32)
    run_case(d, "pm1e4")


@pytest.mark.parametrize("kind", ["nan", "posinf", "allneginf", "token_hi", "token_neg"])
def test_invalid_blocks(kind):
    d = synth.chain_inputs(4, 3, 1030, "f32", T=1.0, seed=12)
    if kind == "nan":
        d["draft"][1, 2, 5] = np.nan
    elif kind == "posinf":
        d["target"][1, 3, 0] = np.inf
    elif kind == "allneginf":
        d["target"][1, 0, :] = -np.inf
    elif kind == "token_hi":
        d["draft_tokens"][1, 2] = 1030
    else:
        d["draft_tokens"][1, 0] = -1
    g, o = run_case(d, f"invalid-{kind}")
    assert o["accept_len"][1] == -1
    assert g["accept_len"][1] == -1 and (g["out_tokens"][1] == -1).all()
    assert (g["accept_len"][[0, 2, 3]] >= 0).all()


@pytest.mark.parametrize("how", ["logit", "temperature"])
def test_outside_library_domain(how):
    """The library restricts rows to |largest finite logit| / T <= 2^28 and
    flags a block with a row beyond it -1.  The oracle evaluates such rows
    (they are nearly one-hot in fp32, so it returns a real outcome), and the
    comparison counts these blocks apart: they must be flagged, never
    matched."""
    if how == "logit":
        d = synth.chain_inputs(4, 3, 1030, "f32", T=1.0, seed=12)
        d["draft"][1, 1, 3] = 3.0e8
    else:
        d = synth.chain_inputs(4, 3, 1030, "f32", T=1e-6, seed=12)
        d["target"][1, 2] += np.float32(300.0)
    g, o = run_case(d, f"domain-{how}")
    assert o["accept_len"][1] >= 0  # the oracle has no such restriction
    assert g["accept_len"][1] == -1 and (g["out_tokens"][1] == -1).all()
    assert (g["accept_len"][[0, 2, 3]] >= 0).all()


def test_uniform_extremes():
    d = synth.chain_inputs(20, 3, 2500, "bf16", T=1.0, seed=13)
    V = d["V"]
    top = np.nextafter(np.float32(1), np.float32(0))
    # The draw's uniform at 0 or just below 1 lies within the band of the
    # CDF's end points, so the comparison checks these blocks against the
    # outcomes admissible there; the assertions pin the exact tokens as well.
    # u = 0 everywhere: every test passes (each p_i(x_i) > 0 here), and the
    # bonus draw takes the first token of positive probability under
    # p_gamma, token 0 (every logit is finite and moderate).
    d["uniforms"] = np.zeros_like(d["uniforms"])
    g, _ = run_case(d, "u0")
    assert (g["accept_len"] == 3).all() and (g["out_tokens"][:, 3] == 0).all()
    # tests at u = 0, the draw at the largest float below 1: the bonus draw
    # takes the last token, V - 1
    d["uniforms"] = np.zeros_like(d["uniforms"])
    d["uniforms"][:, 3] = top
    g, _ = run_case(d, "u-draw-top")
    assert (g["accept_len"] == 3).all() and (g["out_tokens"][:, 3] == V - 1).all()
    # every uniform at the top: a test then passes only where r_i rounds to
    # 1, which lies inside the boundary band (the run must still complete
    # and agree wherever the band allows a comparison)
    d["uniforms"] = np.full_like(d["uniforms"], top)
    run_case(d, "u-top")


def test_repeated_calls_share_workspace():
    """The workspace is scratch: repeated calls on one workspace, refilled with
    garbage bytes in between, agree with each other and with the oracle."""
    torch, sv = require_gpu()
    d = synth.chain_inputs(9, 7, 20000, "bf16", T=0.7, seed=14)
    ws = torch.full((sv.spec_verify_chain_workspace_bytes(9, 7, 20000, sv.SV_DTYPE_BF16),),
                    0xA5, dtype=torch.uint8, device="cuda")
    first = gpu_chain(d, workspace=ws)
    o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                     dtype=d["dtype"])
    compare_chain(first, o, "reuse-first", d=d)
    for fill in (0x00, 0xFF, 0x7F):
        ws.fill_(fill)
        again = gpu_chain(d, workspace=ws)
        assert np.array_equal(first["accept_len"], again["accept_len"])
        assert np.array_equal(first["out_tokens"], again["out_tokens"])


def test_acceptance_frequency_matches_sum_min():
    """Per-position pass rate against sum_v min(p, q) (z-test over blocks)."""
    d = synth.chain_inputs(2000, 4, 600, "f32", T=0.8, target=("normal", 1.5), noise=0.6, seed=15)
    g = gpu_chain(d)
    alpha = oracle.chain_alpha(d["target"], d["draft"], d["T"])
    k = g["accept_len"]
    for i in range(4):
        reached = k >= i
        a = alpha[reached, i]
        sd = np.sqrt((a * (1 - a)).sum())
        assert abs((k[reached] > i).sum() - a.sum()) < 4.5 * sd, i


def test_first_token_chi_square():
    """gamma = 1: the first committed token must follow p_0 (chi-square)."""
    from scipy.special import softmax
    from scipy.stats import chisquare

    rng = np.random.default_rng(16)
    V, B = 32, 100_000
    zp = rng.normal(0, 1.0, (2, V)).astype(np.float32)
    zq = (zp[0] + rng.normal(0, 0.8, V)).astype(np.float32)
    q = softmax(zq.astype(np.float64))
    d = dict(target=np.broadcast_to(zp, (B, 2, V)).copy(),
             draft=np.broadcast_to(zq[None], (B, 1, V)).copy(),
             draft_tokens=rng.choice(V, size=(B, 1), p=q).astype(np.int32),
             uniforms=rng.random((B, 2), dtype=np.float32), B=B, gamma=1, V=V, dtype="f32", T=1.0)
    g = gpu_chain(d)
    obs = np.bincount(g["out_tokens"][:, 0], minlength=V)
    p = softmax(zp[0].astype(np.float64))
    assert chisquare(obs, B * p).pvalue > 1e-4
