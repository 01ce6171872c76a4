"""Pins of the oracle's draft-side sampler (draft_sample_row): exact
enumeration of its law over a uniform grid, the Gumbel-max construction as an
independent sampler of the same law, closed forms and invalid inputs."""
import numpy as np
import pytest
from scipy import stats

import synth
from oracle import spec_verify_oracle as O


def _softmax_ref(L, T):
    z = np.asarray(L, np.float64) / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


@pytest.mark.parametrize("V,T,seed", [(1, 1.0, 0), (2, 0.5, 1), (5, 1.0, 2), (7, 2.5, 3)])
def test_law_by_enumeration(V, T, seed):
    """Over u at the midpoints of K equal cells of [0, 1), the fraction of cells
    that draw v differs from q_v by at most 1/K (the law of the inverse CDF)."""
    g = np.random.default_rng(seed)
    L = g.normal(0, 2, V)
    K = 1 << 14
    counts = np.zeros(V)
    for k in range(K):
        r = O.draft_sample_row(L, T, (k + 0.5) / K)
        counts[r.y] += 1
    q = _softmax_ref(L, T)
    assert np.abs(counts / K - q).max() <= 1.0 / K + 1e-12


def test_matches_gumbel_max_sampler():
    """Chi-square of 20000 inverse-CDF draws at independent uniforms against
    20000 Gumbel-max draws (a different construction of the same law)."""
    g = np.random.default_rng(7)
    V, T = 12, 0.8
    L = g.normal(0, 1.5, V)
    n = 20000
    a = np.bincount([O.draft_sample_row(L, T, float(u)).y for u in g.random(n)], minlength=V)
    gg = np.random.default_rng(8)
    b = np.bincount([synth.gumbel_max_draw(gg, L, T) for _ in range(n)], minlength=V)
    keep = (a + b) > 0
    _, p, _, _ = stats.chi2_contingency(np.stack([a[keep], b[keep]]))
    assert p > 1e-3


def test_closed_forms():
    # equal logits: token floor(u * V)
    V = 10
    for k in range(V):
        assert O.draft_sample_row(np.zeros(V), 1.0, (k + 0.5) / V).y == k
    # one finite logit: that token with probability 1
    L = np.full(9, -np.inf)
    L[6] = 3.0
    r = O.draft_sample_row(L, 0.7, 0.999)
    assert r.y == 6 and r.q_y == 1.0
    # small temperature with a clear maximum: the argmax unless u lies within
    # the (astronomically small) mass of another token
    L = np.array([0.0, 1.0, 5.0, 4.0])
    for u in (1e-6, 0.5, 0.999999):
        assert O.draft_sample_row(L, 0.01, u).y == 2
    # u = 0 draws the first token of positive mass (here e^-500 in fp64)
    assert O.draft_sample_row(L, 0.01, 0.0).y == 0
    # -inf tokens are never drawn, even at u = 0
    L = np.array([-np.inf, -np.inf, 1.0, -np.inf, 2.0])
    assert O.draft_sample_row(L, 1.0, 0.0).y == 2
    # q_y is the tempered softmax at y
    g = np.random.default_rng(3)
    L = g.normal(0, 2, 50)
    r = O.draft_sample_row(L, 1.3, 0.37)
    assert abs(r.q_y - _softmax_ref(L, 1.3)[r.y]) < 1e-15


def test_same_rule_as_the_bonus_draw():
    """With draft rows equal to the target's, every draft is accepted and the
    verify draws the bonus token from target row gamma at u[gamma]: the same
    token the draft sampler draws from that row."""
    g = np.random.default_rng(11)
    for _ in range(20):
        G, V, T = 3, 40, float(g.uniform(0.4, 2.0))
        Lt = g.normal(0, 2, (G + 1, V))
        x = [O.draft_sample_row(Lt[i], T, float(g.random())).y for i in range(G)]
        u = g.random(G + 1)
        res = O.verify_sample_sequence(Lt, Lt[:G].copy(), x, u, T)
        assert res.n == G
        assert res.y == O.draft_sample_row(Lt[G], T, float(u[G])).y


@pytest.mark.parametrize("L,T,u", [
    (np.array([0.0, np.nan]), 1.0, 0.5), (np.array([0.0, np.inf]), 1.0, 0.5),
    (np.full(3, -np.inf), 1.0, 0.5), (np.zeros(3), 0.0, 0.5), (np.zeros(3), np.nan, 0.5),
    (np.zeros(3), 1e-40, 0.5), (np.zeros(3), 1.0, 1.0), (np.zeros(3), 1.0, -0.25)])
def test_invalid(L, T, u):
    r = O.draft_sample_row(L, T, u)
    assert not r.valid and r.y == -1 and np.isnan(r.q_y)


def test_workload_rows():
    d = synth.make_draft_rows(4, 1000, "bf16", T=[0.5, 1.0, 1.5, 2.0], seed=1)
    assert d.logits.dtype == np.uint16 and d.logits.shape == (4, 1000)
    assert ((d.uniforms >= 0) & (d.uniforms < 1)).all()
    assert np.array_equal(d.uniforms, np.round(d.uniforms * 2.0 ** 24) / 2.0 ** 24)
    d2 = synth.make_draft_rows(4, 1000, "bf16", T=[0.5, 1.0, 1.5, 2.0], seed=1)
    assert np.array_equal(d.logits, d2.logits)
