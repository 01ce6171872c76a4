"""GPU tests of the draft-tree attention masks (spec_tree_mask) against the
oracle, bit for bit: the configuration-4 trees with their blocks, random,
chain and star trees up to 1024 nodes, invalid parent arrays mixed into a
batch, unaligned mask buffers and partial output requests."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec_verify_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(gpu, parents, blocks=None, relaxed=True, out_mask=None, out_relaxed=None):
    P = torch.from_numpy(np.ascontiguousarray(parents, np.int32)).cuda()
    Bl = torch.from_numpy(np.ascontiguousarray(blocks, np.int32)).cuda() if blocks is not None else None
    m, r, d = gpu.spec_tree_mask(P, Bl, want_relaxed=relaxed and blocks is not None, out_mask=out_mask,
                                 out_relaxed=out_relaxed)
    torch.cuda.synchronize()
    return (m.cpu().numpy() if m is not None else None, r.cpu().numpy() if r is not None else None,
            d.cpu().numpy() if d is not None else None)


def _check(parents, blocks, got, name):
    m, r, d = got
    bad = 0
    for b in range(parents.shape[0]):
        wm, wr, wd = O.tree_masks(parents[b], blocks[b] if blocks is not None else None)
        ok = np.array_equal(m[b], wm) and np.array_equal(d[b], wd)
        if r is not None:
            ok = ok and np.array_equal(r[b], wr)
        bad += not ok
    H.log(f"[masks {name}] trees={parents.shape[0]} N={parents.shape[1]} mismatches={bad}")
    assert bad == 0


def _random_parents(g, B, N, kind):
    P = np.empty((B, N), np.int32)
    for b in range(B):
        if kind == "chain":
            P[b] = np.arange(-1, N - 1)
        elif kind == "star":
            P[b] = [-1] + [0] * (N - 1)
        else:
            P[b] = [-1] + [int(g.integers(max(0, j - 8) if kind == "deep" else 0, j)) for j in range(1, N)]
    return P


def test_config4_trees_with_blocks(gpu):
    ti = synth.make_tree_inputs(4, seed=0)
    blocks = np.stack([synth.tree_blocks(p) for p in ti.parents])
    _check(ti.parents, blocks, _run(gpu, ti.parents, blocks), "config 4")


@pytest.mark.parametrize("N,kind", [(1, "random"), (2, "random"), (17, "random"), (60, "deep"), (255, "random"),
                                    (353, "deep"),
                                    (1024, "random"), (1024, "chain"), (1024, "star"), (1024, "deep")])
def test_random_trees(gpu, N, kind):
    g = np.random.default_rng(N)
    B = 3 if N >= 255 else 8
    P = _random_parents(g, B, N, kind)
    blocks = g.integers(-1, max(2, N // 3), (B, N)).astype(np.int32)
    _check(P, blocks, _run(gpu, P, blocks), f"{kind} N={N}")


def test_invalid_trees_in_a_batch(gpu):
    g = np.random.default_rng(3)
    P = _random_parents(g, 6, 40, "random")
    P[1, 0] = 0          # root with a parent
    P[3, 17] = 17        # self parent
    P[4, 5] = 30         # forward parent
    P[5, 9] = -1         # second root
    got = _run(gpu, P, np.zeros_like(P))
    _check(P, np.zeros_like(P), got, "invalid mixed")
    assert (got[2][[1, 3, 4, 5]] == -1).all() and not got[0][[1, 3, 4, 5]].any()


def test_unaligned_buffers_and_partial_outputs(gpu):
    g = np.random.default_rng(4)
    P = _random_parents(g, 5, 37, "random")
    Bl = g.integers(-1, 10, P.shape).astype(np.int32)
    n = 5 * 37 * 37
    big = torch.full((n + 64,), 7, dtype=torch.uint8, device="cuda")
    big2 = torch.full((n + 64,), 7, dtype=torch.uint8, device="cuda")
    om = big[3:3 + n].view(5, 37, 37)
    orx = big2[13:13 + n].view(5, 37, 37)
    Pt = torch.from_numpy(P).cuda()
    gpu.spec_tree_mask(Pt, torch.from_numpy(Bl).cuda(), want_relaxed=True, out_mask=om, out_relaxed=orx)
    torch.cuda.synchronize()
    d = gpu.spec_tree_mask(Pt, want_mask=False)[2].cpu().numpy()
    _check(P, Bl, (om.cpu().numpy(), orx.cpu().numpy(), d), "unaligned")
    # bytes around the outputs untouched
    bb, bb2 = big.cpu().numpy(), big2.cpu().numpy()
    assert (bb[:3] == 7).all() and (bb[3 + n:] == 7).all() and (bb2[:13] == 7).all() and (bb2[13 + n:] == 7).all()


@pytest.mark.parametrize("N", [16, 48, 64, 208, 512])
def test_rows_of_whole_vectors(gpu, N):
    """N a multiple of 16 with 16-byte aligned outputs (both masks from one
    pass over the slab), with each mask also requested alone and one invalid
    tree in the batch (its masks all zero)."""
    g = np.random.default_rng(100 + N)
    P = _random_parents(g, 4, N, "random")
    P[2, N // 2] = N // 2 + 1  # forward parent: invalid tree
    Bl = g.integers(-1, max(2, N // 5), P.shape).astype(np.int32)
    _check(P, Bl, _run(gpu, P, Bl), f"whole vectors N={N}")
    Pt, Bt = torch.from_numpy(P).cuda(), torch.from_numpy(Bl).cuda()
    m_only = gpu.spec_tree_mask(Pt, Bt, want_relaxed=False)
    r_only = gpu.spec_tree_mask(Pt, Bt, want_mask=False, want_relaxed=True, want_depth=False)
    torch.cuda.synchronize()
    assert m_only[1] is None and r_only[0] is None and r_only[2] is None
    m, d, r = m_only[0].cpu().numpy(), m_only[2].cpu().numpy(), r_only[1].cpu().numpy()
    for b in range(P.shape[0]):
        wm, wr, wd = O.tree_masks(P[b], Bl[b])
        assert np.array_equal(m[b], wm) and np.array_equal(d[b], wd) and np.array_equal(r[b], wr), b
    assert not m[2].any() and not r[2].any() and (d[2] == -1).all()
