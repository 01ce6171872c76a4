"""Pins of the oracle's draft-tree masks: the ancestor mask equals the
reflexive-transitive closure of the parent relation computed by boolean matrix
powers (an independent algorithm), closed forms for chains and stars, depth
from the mask, the relaxed mask's block structure, and invalid parent arrays."""
import numpy as np
import pytest

import synth
from oracle import spec_verify_oracle as O


def _closure(parents):
    N = len(parents)
    A = np.zeros((N, N), dtype=np.int64)
    for j in range(1, N):
        A[j, parents[j]] = 1
    R = np.eye(N, dtype=np.int64)
    Pk = np.eye(N, dtype=np.int64)
    for _ in range(N):
        Pk = np.minimum(Pk @ A, 1)
        R = np.minimum(R + Pk, 1)
    return R.astype(np.uint8)


@pytest.mark.parametrize("seed", range(6))
def test_mask_is_transitive_closure(seed):
    g = np.random.default_rng(seed)
    N = int(g.integers(1, 40))
    parents = np.array([-1] + [int(g.integers(0, j)) for j in range(1, N)], dtype=np.int32)
    mask, _, depth = O.tree_masks(parents)
    assert np.array_equal(mask, _closure(parents))
    assert np.array_equal(depth, mask.sum(axis=1).astype(np.int32) - 1)


def test_draft_trees_and_blocks():
    g = synth.gen(0, 4, 2, 0)
    parents = synth.tree_shape(g, 60)
    blk = synth.tree_blocks(parents, 2)
    mask, relaxed, depth = O.tree_masks(parents, blk)
    assert np.array_equal(mask, _closure(parents))
    # blocks are 2-node chains (cut trees may end a block early): ids repeat at most twice
    ids, counts = np.unique(blk[1:], return_counts=True)
    assert counts.max() <= 2 and (blk[0] == -1)
    # the relaxed mask adds exactly the later member of a block to the earlier one's row
    extra = relaxed.astype(int) - mask.astype(int)
    assert extra.min() == 0
    for i, j in zip(*np.nonzero(extra)):
        assert blk[i] == blk[j] and blk[i] >= 0 and parents[j] == i
    for k in ids[counts == 2]:
        a, b = np.flatnonzero(blk == k)
        assert relaxed[a, b] == relaxed[b, a] == 1 and mask[a, b] == 0


def test_closed_forms():
    N = 7
    chain = np.arange(-1, N - 1, dtype=np.int32)
    m, _, d = O.tree_masks(chain)
    assert np.array_equal(m, np.tril(np.ones((N, N), np.uint8))) and list(d) == list(range(N))
    star = np.array([-1] + [0] * (N - 1), dtype=np.int32)
    m, _, d = O.tree_masks(star)
    want = np.eye(N, dtype=np.uint8)
    want[:, 0] = 1
    assert np.array_equal(m, want) and list(d) == [0] + [1] * (N - 1)
    m, r, d = O.tree_masks(np.array([-1], np.int32), np.array([-1], np.int32))
    assert m.tolist() == [[1]] and r.tolist() == [[1]] and d.tolist() == [0]


@pytest.mark.parametrize("parents", [[0, 0], [-1, 1], [-1, 0, 3, 1], [-1, -1], [5]])
def test_invalid(parents):
    m, r, d = O.tree_masks(np.array(parents, np.int32), np.zeros(len(parents), np.int32))
    assert not m.any() and not r.any() and (d == -1).all()


def test_nodes_without_a_block_see_only_their_path():
    """Block id -1 means 'no block': with no blocks at all the relaxed mask is
    the tree mask, and two unblocked nodes never see each other through it."""
    g = np.random.default_rng(9)
    N = 25
    parents = np.array([-1] + [int(g.integers(0, j)) for j in range(1, N)], dtype=np.int32)
    mask, relaxed, _ = O.tree_masks(parents, np.full(N, -1, np.int32))
    assert np.array_equal(relaxed, mask)
    blocks = np.where(np.arange(N) % 3 == 0, -1, np.arange(N) // 6).astype(np.int32)
    mask, relaxed, _ = O.tree_masks(parents, blocks)
    for i in range(N):
        for j in range(N):
            if blocks[i] == -1 or blocks[j] == -1:
                assert relaxed[i, j] == mask[i, j]
