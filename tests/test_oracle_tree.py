"""Pins of the greedy tree oracle: brute force over small trees and the greedy walk."""
import itertools

import numpy as np

from oracle import spec_verify_oracle as O


def _all_parent_arrays(N):
    """Every parent array with parents[0] = -1 and 0 <= parents[j] < j."""
    for rest in itertools.product(*[range(j) for j in range(1, N)]):
        yield [-1] + list(rest)


def _brute_force(L, parents, tokens):
    """Enumerate every root path; keep those whose every edge matches the parent's
    top token; the deepest wins, lowest end node on ties."""
    N, V = L.shape
    g = [int(np.argmax(L[j])) for j in range(N)]
    best = (0, 0)  # (depth, -node)
    for end in range(N):
        path = []
        k = end
        while k != -1:
            path.append(k)
            k = parents[k]
        path.reverse()
        ok = all(tokens[path[i + 1]] == g[path[i]] for i in range(len(path) - 1))
        if ok and (len(path) - 1, -end) > best:
            best = (len(path) - 1, -end)
    d = -best[1]
    path = []
    k = d
    while k != -1:
        path.append(k)
        k = parents[k]
    return best[0], path[::-1], g[d]


def test_exhaustive_small_trees():
    g = np.random.default_rng(0)
    V = 3
    checked = 0
    for N in range(1, 7):
        for parents in _all_parent_arrays(N):
            for _ in range(3):
                L = g.integers(-2, 3, size=(N, V)).astype(np.float64)  # ties are common
                tokens = [0] + list(g.integers(0, V, size=N - 1))
                r = O.verify_tree_sequence(L, parents, tokens)
                assert r.valid
                assert (r.accept_len, r.path, r.bonus) == _brute_force(L, parents, tokens)
                checked += 1
    assert checked > 400


def test_flags_equal_greedy_walk_with_distinct_siblings():
    g = np.random.default_rng(1)
    for _ in range(300):
        N = int(g.integers(2, 30))
        V = 8
        parents = [-1] + [int(g.integers(0, j)) for j in range(1, N)]
        kids = {}
        for j in range(1, N):
            kids.setdefault(parents[j], []).append(j)
        tokens = [0] * N
        for p, ks in kids.items():
            if len(ks) > V:
                break
            for k, t in zip(ks, g.permutation(V)[: len(ks)]):
                tokens[k] = int(t)
        else:
            L = g.normal(size=(N, V))
            # plant matches on most edges so that paths get deep
            for j in range(1, N):
                if g.random() < 0.7:
                    L[parents[j], tokens[j]] = 10.0 + g.random()
            a = O.verify_tree_sequence(L, parents, tokens)
            b = O.greedy_walk(L, parents, tokens)
            assert (a.accept_len, a.path, a.bonus) == (b.accept_len, b.path, b.bonus)


def test_invalid_trees():
    L = np.zeros((3, 4))
    assert not O.verify_tree_sequence(L, [0, 0, 1], [0, 1, 1]).valid  # root parent must be -1
    assert not O.verify_tree_sequence(L, [-1, 1, 1], [0, 1, 1]).valid  # parent must be < j
    assert not O.verify_tree_sequence(L, [-1, 0, 0], [0, 4, 1]).valid  # token out of range
    assert not O.verify_tree_sequence(L, [-1, 0, 0], [0, -1, 1]).valid
    assert O.verify_tree_sequence(L, [-1, 0, 0], [7, 0, 1]).valid  # the root's token is unused
