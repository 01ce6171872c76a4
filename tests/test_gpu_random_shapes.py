"""GPU parity on seeded random shapes: batch, gamma, vocabulary, dtypes,
row padding and per-sequence temperatures drawn at random (fixed seeds), so
that the combinations between the hand-picked edge cases are covered too: the
one-pass call and the early-exit call against the fp64 oracle with the parity
contract, and against each other; greedy trees of random size, vocabulary and
dtype bit for bit; draft-side sampling of random batches (both of its paths:
one pass for many or short rows, statistics and draw for few long ones); tree
masks of random parent arrays and blocks bit for bit; the early exit under a
random grouping of positions."""
import numpy as np
import pytest

import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = 24
TREE_CASES = 8
DRAFT_CASES = 8


def _shape(k):
    g = np.random.default_rng(9000 + k)
    V = int(np.exp(g.uniform(np.log(2), np.log(300000))))
    G = int(g.integers(1, 21))
    B = int(g.integers(1, 41))
    # keep the oracle's work (all rows of every sequence) to a few seconds
    while B > 1 and B * (2 * G + 1) * V > 30_000_000:
        B //= 2
    tdt, ddt = g.choice(["bf16", "f32"], 2)
    pad = None if g.random() < 0.5 else int(-(-V // 8) * 8 + 8 * g.integers(0, 4))
    if pad is None and V % 8:
        pad = -(-V // 8) * 8  # rows must start on 16-byte boundaries (the C ABI rejects others)
    T = g.uniform(0.3, 2.0, B).astype(np.float32)
    return B, G, V, str(tdt), str(ddt), pad, T


@pytest.mark.parametrize("k", range(CASES))
def test_random_shape(gpu, k):
    B, G, V, tdt, ddt, pad, T = _shape(k)
    H.log(f"random shape {k}: B={B} gamma={G} V={V} {tdt}/{ddt} pad={pad}")
    inp = synth.make_custom_sample(B, G, V, tdt, ddt, T=T, noise_sd=0.6, seed=k + 1)
    tens = H.sample_tensors(inp, pad_to=pad)
    one = H.run_sample(gpu, tens)
    ee = H.run_sample(gpu, tens, early_exit=True)
    for name, out in (("one pass", one), ("early exit", ee)):
        t = H.check_sample(inp, out)
        H.log(f"[random {k} {name}] {t.summary()}")
        assert not t.fail, t.fail[:3]
        assert t.flagged <= 2
    differ, bad = H.compare_one_pass(one, ee)
    assert not bad, bad[:3]


@pytest.mark.parametrize("k", range(TREE_CASES))
def test_random_tree_shape(gpu, k):
    g = np.random.default_rng(9500 + k)
    B = int(g.integers(1, 17))
    N = int(np.exp(g.uniform(0, np.log(120))))  # the draft-tree generator reaches ~120 nodes at depth 6
    V = int(np.exp(g.uniform(np.log(8), np.log(200000))))
    while B > 1 and B * N * V > 30_000_000:
        B //= 2
    V = -(-V // 8) * 8  # whole 16-byte rows for either dtype
    dt = str(g.choice(["bf16", "f32"]))
    H.log(f"random tree shape {k}: B={B} N={N} V={V} {dt}")
    ti = synth.make_tree_inputs(4, seed=k + 1, B=B, N=N, V=V, dtype=dt)
    out = H.run_tree(gpu, H.tree_tensors(ti))
    fails = H.check_tree(ti.logits, ti.dtype, ti.parents, ti.tokens, out)
    H.log(f"[random tree {k}] trees={B} mismatches={len(fails)}")
    assert not fails, fails[:3]


@pytest.mark.parametrize("k", range(DRAFT_CASES))
def test_random_draft_shape(gpu, k):
    g = np.random.default_rng(9700 + k)
    B = int(np.exp(g.uniform(0, np.log(300))))
    V = int(np.exp(g.uniform(np.log(2), np.log(400000))))
    while B > 1 and B * V > 30_000_000:
        B //= 2
    dt = str(g.choice(["bf16", "f32"]))
    T = g.uniform(0.3, 2.0, B).astype(np.float32)
    H.log(f"random draft shape {k}: B={B} V={V} {dt}")
    d = synth.make_draft_rows(B, V, dt, T=T, seed=k + 1)
    t = H.check_draft(d, H.run_draft(gpu, H.draft_tensors(d, pad_to=-(-V // 8) * 8 if V % 8 else None)))
    H.log(f"[random draft {k}] {t.summary()}")
    assert not t.fail, t.fail[:3]
    assert t.flagged <= 2


MASK_CASES = 8


@pytest.mark.parametrize("k", range(MASK_CASES))
def test_random_mask_shape(gpu, k):
    """spec_tree_mask on random parent arrays (N from 1 to 300, on both sides
    of the one-wave kernel's 64 nodes; parents at most w back, w random), random
    block ids and, now and then, an invalid tree in the batch: bit-exact
    against the oracle."""
    import torch

    from oracle import spec_verify_oracle as O

    g = np.random.default_rng(9900 + k)
    B = int(g.integers(1, 9))
    N = int(np.exp(g.uniform(0, np.log(300))))
    P = np.empty((B, N), np.int32)
    for b in range(B):
        w = int(g.integers(1, 20))
        P[b] = [-1] + [int(g.integers(max(0, j - w), j)) for j in range(1, N)]
    if B > 1 and N > 2 and g.random() < 0.5:
        P[B - 1, N - 1] = N - 1  # a self parent: invalid tree
    Bl = g.integers(-1, max(2, N // 3), (B, N)).astype(np.int32)
    H.log(f"random mask shape {k}: B={B} N={N}")
    m, r, d = gpu.spec_tree_mask(torch.from_numpy(P).cuda(), torch.from_numpy(Bl).cuda(), want_relaxed=True)
    torch.cuda.synchronize()
    m, r, d = m.cpu().numpy(), r.cpu().numpy(), d.cpu().numpy()
    for b in range(B):
        wm, wr, wd = O.tree_masks(P[b], Bl[b])
        assert np.array_equal(m[b], wm) and np.array_equal(r[b], wr) and np.array_equal(d[b], wd), (k, b)


@pytest.mark.parametrize("k", range(8))
def test_random_shape_grouped_early_exit(gpu, k):
    """The early exit with a random grouping of positions (tail start 0..gamma)
    on random shapes, against the oracle and the one-pass call."""
    g = np.random.default_rng(9800 + k)
    V = int(np.exp(g.uniform(np.log(1), np.log(300000))))
    G = int(g.integers(1, 20))
    B = int(g.integers(1, 60))
    while B > 1 and B * (2 * G + 1) * V > 20_000_000:
        B //= 2
    tdt, ddt = [str(x) for x in g.choice(["bf16", "f32"], 2)]
    pad = -(-V // 8) * 8 if V % 8 else None
    ts = int(g.integers(0, G + 1))
    H.log(f"random grouped early exit {k}: B={B} gamma={G} V={V} {tdt}/{ddt} tail_start={ts}")
    inp = synth.make_custom_sample(B, G, V, tdt, ddt, T=g.uniform(0.3, 2.0, B).astype(np.float32),
                                   noise_sd=float(g.uniform(0.05, 1.5)), seed=k + 101)
    tens = H.sample_tensors(inp, pad_to=pad)
    one = H.run_sample(gpu, tens)
    ee = H.run_sample(gpu, tens, early_exit=True, tail_start=ts)
    for name, out in (("one pass", one), ("early exit", ee)):
        t = H.check_sample(inp, out)
        H.log(f"[random grouped {k} {name}] {t.summary()}")
        assert not t.fail, t.fail[:3]
        assert t.flagged <= max(2, 0.01 * t.checked)
    differ, bad = H.compare_one_pass(one, ee)
    assert not bad, bad[:3]
