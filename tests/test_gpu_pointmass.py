"""GPU parity of spec_verify_chain_pointmass against the fp64 oracle (needs an
MI355X).  Same comparison rule as the chain: exact accept lengths and tokens
outside the 1e-6 boundary band, final_dist to 1e-5."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_chain, gpu_chain, gpu_pointmass, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_case(d, label, want_dist=True):
    print(f"[case] {label} B={d['B']} gamma={d['gamma']} V={d['V']} {d['dtype']} T={d['T']}",
          flush=True)
    g = gpu_pointmass(d, want_dist=want_dist)
    o = oracle.chain_pointmass(d["target"], d["draft_tokens"], d["uniforms"], d["T"],
                               dtype=d["dtype"], want_dist=want_dist)
    n, near = compare_chain(g, o, label, d=d, pointmass=True)
    print(f"[case] {label}: compared {n} blocks, {near} inside the boundary band", flush=True)
    return g, o


SHAPES = [(3, 1, 1), (5, 2, 7), (4, 31, 1000), (2, 3, 5003), (1, 16, 151937), (7, 4, 4096),
          (2, 255, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}g{g}V{v}" for b, g, v in SHAPES])
def test_shapes_and_ragged_tails(shape, dtype):
    B, g, V = shape
    for seed in range(3):
        d = synth.pointmass_inputs(B, g, V, dtype, T=0.9, target=("normal", 2.0), p_match=0.7,
                                   seed=2000 + seed)
        run_case(d, f"pm-shape{shape}-{dtype}-s{seed}")


# Large batches: each final-draw workgroup streams a run of several tiles
# (runs of 2 to 17 tiles, ragged last tile, unaligned rows).
LONG_SHAPES = [(256, 3, 40000, "bf16"), (512, 1, 65541, "bf16"), (300, 2, 20003, "f32")]


@pytest.mark.parametrize("shape", LONG_SHAPES, ids=[f"B{b}g{g}V{v}{t}" for b, g, v, t in LONG_SHAPES])
def test_long_chunk_runs(shape):
    B, g, V, dtype = shape
    d = synth.pointmass_inputs(B, g, V, dtype, T=0.8, target=("normal", 2.0), p_match=0.7,
                               seed=4200 + g)
    run_case(d, f"pm-long{shape}")


# 20 seeded rounds each of the point-mass workloads with the shapes of
# configs 3 and 5 (final_dist compared on every one), in chunks that keep each
# test well under a minute.
PM_FULL = ([(3, range(i, i + 5)) for i in range(0, 20, 5)] +
           [(5, range(i, i + 4)) for i in range(0, 20, 4)])


@pytest.mark.parametrize("cfg,seeds", PM_FULL,
                         ids=[f"pm{c}-s{r.start}-{r.stop - 1}" for c, r in PM_FULL])
def test_config_shapes_full_size(cfg, seeds):
    for s in seeds:
        d = synth.pointmass_config_inputs(cfg, seed=7000 + 10 * s + cfg)
        run_case(d, f"pm-config{cfg}-s{s}", want_dist=True)


def test_more_uniforms_config3():
    d = synth.pointmass_config_inputs(3, seed=7100)
    rng = np.random.default_rng(71)
    for r in range(3):
        d["uniforms"] = rng.random(d["uniforms"].shape, dtype=np.float32)
        run_case(d, f"pm-config3-u{r}", want_dist=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_same_as_chain_with_one_hot_draft(dtype):
    """With one-hot draft logits the chain's ratio test and residual reduce to
    the point-mass rule: both entry points give identical outputs."""
    d = synth.pointmass_inputs(40, 5, 3001, dtype, T=0.8, seed=31)
    ninf = np.float32(-np.inf) if dtype == "f32" else np.uint16(0xFF80)
    zero = np.float32(0.0) if dtype == "f32" else np.uint16(0)
    drf = np.full((40, 5, 3001), ninf, dtype=d["target"].dtype)
    for b in range(40):
        drf[b, np.arange(5), d["draft_tokens"][b]] = zero
    c = dict(d, draft=drf)
    a = gpu_chain(c)
    pm = gpu_pointmass(d)
    assert np.array_equal(a["accept_len"], pm["accept_len"])
    assert np.array_equal(a["out_tokens"], pm["out_tokens"])


@pytest.mark.parametrize("kind", ["nan", "posinf", "allneginf", "token_hi", "token_neg"])
def test_invalid_blocks(kind):
    d = synth.pointmass_inputs(4, 3, 1030, "f32", T=1.0, seed=12)
    if kind == "nan":
        d["target"][1, 2, 5] = np.nan
    elif kind == "posinf":
        d["target"][1, 3, 0] = np.inf
    elif kind == "allneginf":
        d["target"][1, 0, :] = -np.inf
    elif kind == "token_hi":
        d["draft_tokens"][1, 2] = 1030
    else:
        d["draft_tokens"][1, 0] = -1
    g, _ = run_case(d, f"pm-invalid-{kind}")
    assert g["accept_len"][1] == -1 and (g["out_tokens"][1] == -1).all()
    assert (g["accept_len"][[0, 2, 3]] >= 0).all()


def test_masked_and_certain_tokens():
    """A masked draft token (p = 0) is always rejected and never drawn; a token
    holding all of its row's mass is always accepted."""
    d = synth.pointmass_inputs(16, 4, 2000, "bf16", T=1.0, seed=33)
    tok = d["draft_tokens"]
    for b in range(8):
        d["target"][b, 0, tok[b, 0]] = 0xFF80  # -inf
    for b in range(8, 16):
        d["target"][b, 0, :] = 0xFF80
        d["target"][b, 0, tok[b, 0]] = 0
    g, o = run_case(d, "pm-masked-certain")
    assert (g["accept_len"][:8] == 0).all()
    assert all(g["out_tokens"][b, 0] != tok[b, 0] for b in range(8))
    assert (g["accept_len"][8:] >= 1).all()


def test_acceptance_frequency():
    """Per-position pass rate against p_i(x_i) (z-test over blocks)."""
    from scipy.special import softmax

    d = synth.pointmass_inputs(3000, 3, 300, "f32", T=0.8, target=("normal", 1.0), p_match=0.6,
                               seed=34)
    g = gpu_pointmass(d)
    k = g["accept_len"]
    p = softmax(d["target"].astype(np.float64) / 0.8, axis=2)
    px = np.take_along_axis(p[:, :3], d["draft_tokens"][:, :, None], axis=2)[..., 0]
    for i in range(3):
        reached = k >= i
        a = px[reached, i]
        sd = np.sqrt((a * (1 - a)).sum())
        assert abs((k[reached] > i).sum() - a.sum()) < 4.5 * sd, i


def test_uniform_extremes():
    """Draws at the ends of the CDF (uniform 0, or the largest float below 1)
    sit within the band of the CDF's end points, so the oracle comparison
    excludes them; the assertions pin them: the first and the last token of
    positive weight."""
    d = synth.pointmass_inputs(20, 3, 2500, "bf16", T=1.0, seed=35)
    V = d["V"]
    tok = d["draft_tokens"]
    top = np.nextafter(np.float32(1), np.float32(0))
    # every test passes at u = 0 (each p_i(x_i) > 0); the bonus draw takes
    # token 0 at u = 0 and token V - 1 just below 1
    for u_draw, want in ((0.0, 0), (top, V - 1)):
        d["uniforms"] = np.zeros_like(d["uniforms"])
        d["uniforms"][:, 3] = u_draw
        g, _ = run_case(d, f"pm-accept-draw{u_draw:.0f}")
        assert (g["accept_len"] == 3).all() and (g["out_tokens"][:, 3] == want).all()
    # the first test fails just below 1 (no p_0(x_0) is that close to 1
    # here); the draw from p_0 without x_0 then takes the first or the last
    # token other than x_0
    for u_draw, want in ((0.0, np.where(tok[:, 0] == 0, 1, 0)),
                         (top, np.where(tok[:, 0] == V - 1, V - 2, V - 1))):
        d["uniforms"] = np.zeros_like(d["uniforms"])
        d["uniforms"][:, 0] = top
        d["uniforms"][:, 3] = u_draw
        g, _ = run_case(d, f"pm-reject-draw{u_draw:.0f}")
        assert (g["accept_len"] == 0).all() and (g["out_tokens"][:, 0] == want).all()


@pytest.mark.parametrize("dtype,g,V,mult", [("bf16", 4, 151936, 1.0), ("f32", 4, 151936, 1.0),
                                            ("bf16", 255, 4096, 1.0), ("bf16", 3, 40000, 2.2)])
def test_block_draw_matches_chunk_draw(dtype, g, V, mult):
    """A point-mass batch of at least one block per compute unit draws each
    block in one workgroup (quarter sums kept in LDS), a smaller batch in
    chunk workgroups and a selection kernel.  Both form the same quarter sums
    and select the same way, and blocks are independent, so each block must
    give bit-identical accept lengths, tokens and final_dist whether the whole
    batch goes in one call (one workgroup per block) or in calls of fewer
    blocks than compute units (chunks).  gamma = 255 also takes the outputs'
    writes past the first wave's 64 lanes; 2.2 blocks per compute unit runs
    the one-workgroup-per-block kernel over several rounds."""
    torch, _ = require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B = int(cus * mult)
    d = synth.pointmass_inputs(B, g, V, dtype, T=0.8, target=("gumbel", 4.0), p_match=0.8,
                               seed=4300 + g)
    print(f"[case] pm block-vs-chunk B={B} gamma={g} V={V} {dtype}", flush=True)
    whole = gpu_pointmass(d, want_dist=True)
    part = max(1, cus - 1)
    pieces = []
    for b0 in range(0, B, part):
        sub = {k: (v[b0:b0 + part] if isinstance(v, np.ndarray) and v.shape[:1] == (B,) else v)
               for k, v in d.items()}
        sub["B"] = len(sub["draft_tokens"])
        pieces.append(gpu_pointmass(sub, want_dist=True))
    for key in ("accept_len", "out_tokens", "final_dist"):
        assert np.array_equal(whole[key], np.concatenate([p_[key] for p_ in pieces])), key
    # the batch is not degenerate: rejections (residual of p without the
    # rejected token) occur, and for short blocks full acceptances too
    acc = whole["accept_len"]
    assert (acc < g).sum() > 10
    if g < 16:
        assert (acc == g).sum() > 0
