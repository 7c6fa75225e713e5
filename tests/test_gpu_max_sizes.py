"""GPU parity at the largest vocabulary the library accepts (needs an MI355X).

V = 2^29 is the vocabulary limit checked on the host: below it, every 32-bit
element index in the kernels, plus a tile or a segment, stays inside int32.
The rows are seeded pools of bf16 logits tiled to full length, which is cheap
to build at this size. The tokens that decide each case sit near the end of
the rows, so element and byte offsets reach their largest values. Each decision
is far from its boundary, so the oracle comparison covers every block."""
import time

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (compare_chain, compare_tree, gpu_chain, gpu_pointmass, gpu_tree,
                      require_gpu, to_dev, to_dev_logits)

pytestmark = pytest.mark.gpu

POOLS = (1_000_003, 999_983, 1_000_033, 999_979, 1_000_037, 999_961)


def _rows(n, V, seed):
    """n rows of V bf16 logits: seeded N(0, 1) pools of prime lengths, tiled."""
    rng = np.random.default_rng(seed)
    out = np.empty((n, V), np.uint16)
    for r in range(n):
        pool = synth.bf16_bits(rng.standard_normal(POOLS[r % len(POOLS)]).astype(np.float32))
        out[r] = np.resize(pool, V)
    return out


def _bf16(x):
    return synth.bf16_bits(np.array([x], np.float32))[0]


def test_chain_at_the_largest_vocabulary():
    torch, sv = require_gpu()
    V = sv.SV_MAX_VOCAB
    B, g = 2, 1
    t0 = time.time()
    tgt = _rows(2 * B, V, 81).reshape(B, 2, V)
    dr = _rows(B, V, 82).reshape(B, 1, V)
    x = V - 7
    # block 0: target and draft both put most of their mass on x (p(x) ~ 0.8
    # >= q(x) ~ 0.7, so the test passes), and the bonus row puts ~0.8 on
    # V - 3, where the draw at u = 0.9 lands
    tgt[0, 0, x], dr[0, 0, x], tgt[0, 1, V - 3] = _bf16(22.0), _bf16(21.5), _bf16(22.0)
    # block 1: the draft is surer of x than the target (r ~ 0.16, rejected at
    # u = 0.9), and the target's token V - 2 holds most of the residual, where
    # the draw at u = 0.5 lands
    tgt[1, 0, x], dr[1, 0, x], tgt[1, 0, V - 2] = _bf16(20.0), _bf16(21.0), _bf16(22.0)
    d = dict(target=tgt, draft=dr, draft_tokens=np.full((B, g), x, np.int32),
             uniforms=np.array([[0.5, 0.9], [0.9, 0.5]], np.float32), B=B, gamma=g, V=V,
             dtype="bf16", T=1.0)
    print(f"[case] max-V chain B={B} gamma={g} V={V}: inputs in {time.time() - t0:.1f}s", flush=True)
    res = gpu_chain(d)
    print(f"[case] max-V chain: GPU done at {time.time() - t0:.1f}s", flush=True)
    o = oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                     dtype="bf16")
    print(f"[case] max-V chain: oracle done at {time.time() - t0:.1f}s", flush=True)
    n, near = compare_chain(res, o, "max-V chain", check_dist=False, d=d)
    assert n == B and near == 0
    assert res["accept_len"].tolist() == [1, 0]
    assert res["out_tokens"].tolist() == [[x, V - 3], [V - 2, -1]]


def test_tree_at_the_largest_ragged_vocabulary():
    """V = 2^29 - 3: rows are not 16-byte aligned (scalar heads and tails in
    every segment), and each row's argmax sits in its last few elements."""
    torch, sv = require_gpu()
    V = sv.SV_MAX_VOCAB - 3
    t0 = time.time()
    rows = _rows(4, V, 83)
    # root -> 1 -> 2 matches the argmax at every step; node 3 does not; the
    # bonus token is row 2's argmax, the very last element
    rows[0, V - 5], rows[1, V - 4], rows[2, V - 1] = _bf16(9.0), _bf16(9.0), _bf16(9.0)
    d = dict(target=rows.reshape(1, 4, V), parents=np.array([[-1, 0, 1, 0]], np.int32),
             tokens=np.array([[0, V - 5, V - 4, V - 6]], np.int32), dtype="bf16")
    print(f"[case] max-V tree n=4 V={V}: inputs in {time.time() - t0:.1f}s", flush=True)
    res = gpu_tree(d)
    o = oracle.tree_greedy(d["target"], d["parents"], d["tokens"])
    print(f"[case] max-V tree: done at {time.time() - t0:.1f}s", flush=True)
    compare_tree(res, o, "max-V tree")
    assert res["accept_len"].tolist() == [2] and res["accept_node"].tolist() == [2]
    assert res["out_tokens"][0, :3].tolist() == [V - 5, V - 4, V - 1]


def test_pointmass_at_the_largest_vocabulary():
    torch, sv = require_gpu()
    V = sv.SV_MAX_VOCAB
    B, g = 2, 1
    tgt = _rows(2 * B, V, 84).reshape(B, 2, V)
    x = V - 7
    # block 0: p(x) ~ 0.8 passes at u = 0.5; the bonus row's ~0.8 on V - 3
    # takes the draw at u = 0.9.  Block 1: p(x) ~ 0.1 fails at u = 0.9; the
    # draw from p without x lands on V - 2 (~0.8 of what is left) at u = 0.5
    tgt[0, 0, x], tgt[0, 1, V - 3] = _bf16(22.0), _bf16(22.0)
    tgt[1, 0, x], tgt[1, 0, V - 2] = _bf16(20.0), _bf16(22.0)
    d = dict(target=tgt, draft_tokens=np.full((B, g), x, np.int32),
             uniforms=np.array([[0.5, 0.9], [0.9, 0.5]], np.float32), B=B, gamma=g, V=V,
             dtype="bf16", T=1.0)
    print(f"[case] max-V point-mass B={B} gamma={g} V={V}", flush=True)
    res = gpu_pointmass(d)
    o = oracle.chain_pointmass(d["target"], d["draft_tokens"], d["uniforms"], d["T"],
                               dtype="bf16")
    n, near = compare_chain(res, o, "max-V point-mass", check_dist=False, d=d,
                               pointmass=True)
    assert n == B and near == 0
    assert res["accept_len"].tolist() == [1, 0]
    assert res["out_tokens"].tolist() == [[x, V - 3], [V - 2, -1]]



def test_stochastic_tree_at_the_largest_vocabulary():
    torch, sv = require_gpu()
    V = sv.SV_MAX_VOCAB
    n = 3
    tgt = _rows(n, V, 86).reshape(1, n, V)
    dr = _rows(n, V, 87).reshape(1, n, V)
    y1, y2 = V - 7, V - 5
    # node 1 (child of the root): both root rows put most of their mass on y1
    # (p ~ 0.8 >= q ~ 0.7, passes at u = 0.5); node 2 (child of node 1): node
    # 1's draft row is surer of y2 than its target row (r ~ 0.16, fails at
    # u = 0.9).  The correction comes from target row 1, whose ~0.35 on y2
    # takes the draw at u = 0.9
    tgt[0, 0, y1], dr[0, 0, y1] = _bf16(22.0), _bf16(21.5)
    tgt[0, 1, y2], dr[0, 1, y2] = _bf16(20.0), _bf16(21.0)
    par = np.array([[-1, 0, 1]], np.int32)
    tok = np.array([[0, y1, y2]], np.int32)
    uni = np.array([[0.9, 0.5, 0.9]], np.float32)
    print(f"[case] max-V stochastic tree n={n} V={V}", flush=True)
    acc, node, out, _ = sv.spec_verify_tree_stochastic(
        to_dev_logits(tgt, "bf16"), to_dev_logits(dr, "bf16"), to_dev(par, np.int32),
        to_dev(tok, np.int32), to_dev(uni, np.float32), 1.0)
    torch.cuda.synchronize()
    o = oracle.tree_stochastic(tgt, dr, par, tok, uni, 1.0, dtype="bf16")
    assert o["margin"][0] >= 1e-6
    assert acc.cpu().tolist() == o["accept_len"].tolist() == [1]
    assert node.cpu().tolist() == o["accept_node"].tolist() == [1]
    assert out.cpu().tolist() == o["out_tokens"].tolist() == [[y1, y2, -1]]


def test_tree_construction_at_the_largest_vocabulary():
    torch, sv = require_gpu()
    V = sv.SV_MAX_VOCAB
    W, N, budget = 2, 2, 5
    rows = _rows(3, V, 88).reshape(1, 3, V)
    # root row: V - 3 (~0.6) then V - 9 (~0.23); row 1, the child through
    # V - 3 and the best queued node after the root, puts ~0.6 on V - 1 and
    # ~0.23 on V - 2, which fill the budget
    rows[0, 0, V - 3], rows[0, 0, V - 9] = _bf16(22.0), _bf16(21.0)
    rows[0, 1, V - 1], rows[0, 1, V - 2] = _bf16(22.0), _bf16(21.0)
    print(f"[case] max-V tree construction M=3 V={V} W={W} N={N} budget={budget}", flush=True)
    par, tok, row, sc, n = sv.spec_tree_build(to_dev_logits(rows, "bf16"), 1.0, W, N, budget)
    torch.cuda.synchronize()
    o = oracle.tree_build(rows, 1.0, W, N, budget, dtype="bf16")
    assert o["min_gap"][0] >= 1e-4
    assert n.cpu().tolist() == o["n"].tolist() == [5]
    assert par.cpu().tolist() == o["parents"].tolist() == [[-1, 0, 0, 1, 1]]
    assert tok.cpu().tolist() == o["tokens"].tolist() == [[-1, V - 3, V - 9, V - 1, V - 2]]
    assert row.cpu().tolist() == o["rows"].tolist()
    assert np.allclose(sc.cpu().numpy(), o["score"], rtol=0, atol=1e-4)
