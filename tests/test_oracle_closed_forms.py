"""Closed forms and hand-derived cases that the sampling and tree oracles must reproduce."""
import numpy as np
import pytest

from oracle import spec_verify_oracle as O
from tests.golden_io import farray, load


@pytest.mark.parametrize("case", load("sample_cases.json"), ids=lambda c: c["name"])
def test_sample_golden(case):
    r = O.verify_sample_sequence(farray(case["target"]), farray(case["draft"]), case["x"], case["u"], case["T"])
    assert r.valid == case["valid"]
    if not case["valid"]:
        return
    assert r.n == case["n"]
    assert r.tokens == case["tokens"]
    assert r.resid_mass == pytest.approx(case["resid_mass"], rel=1e-12)
    for i, want in enumerate(case["rho"]):
        if want is not None:
            assert r.rho[i] == pytest.approx(want, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("case", load("tree_cases.json"), ids=lambda c: c["name"])
def test_tree_golden(case):
    r = O.verify_tree_sequence(farray(case["logits"]), case["parents"], case["tokens"])
    assert r.valid == case["valid"]
    if case["valid"]:
        assert r.accept_len == case["accept_len"]
        assert r.path == case["path"]
        assert r.bonus == case["bonus"]
        assert list(r.argmax) == case["argmax"]


def _random_rows(g, n, V, sd=2.0):
    return g.normal(0, sd, size=(n, V))


@pytest.mark.parametrize("gamma", [1, 3, 8])
def test_identical_rows_accept_everything(gamma):
    """q == p gives rho = 1 at every position, so every draft is accepted and the
    final token is the bonus draw from the last target row."""
    g = np.random.default_rng(gamma)
    V, T = 40, 0.8
    Lt = _random_rows(g, gamma + 1, V)
    Ld = Lt[:gamma].copy()
    for _ in range(50):
        x = g.integers(0, V, size=gamma)
        u = g.integers(0, 1 << 24, size=gamma + 1) * 2.0 ** -24
        r = O.verify_sample_sequence(Lt, Ld, x, u, T)
        assert r.valid and r.n == gamma and r.bonus
        np.testing.assert_allclose(r.rho, 1.0, rtol=1e-13)
        y_ref, _, _ = O.inverse_cdf(O.tempered_softmax(Lt[gamma], T)[0], u[gamma])
        assert r.tokens == list(x) + [y_ref]


def test_disjoint_supports_reject_at_zero():
    """p and q with disjoint supports: rho_0 = 0, so position 0 always rejects,
    and the residual max(0, p_0 - q_0) is p_0 itself: y is an exact draw from p_0."""
    g = np.random.default_rng(11)
    V, gamma, T = 30, 4, 1.3
    for _ in range(40):
        Lt = _random_rows(g, gamma + 1, V)
        Ld = _random_rows(g, gamma, V)
        half = g.permutation(V)
        A, Bs = half[: V // 2], half[V // 2:]
        Lt[0, Bs] = -np.inf
        Ld[0, A] = -np.inf
        x = [int(g.choice(Bs))] + list(g.integers(0, V, size=gamma - 1))
        u = g.integers(0, 1 << 24, size=gamma + 1) * 2.0 ** -24
        r = O.verify_sample_sequence(Lt, Ld, x, u, T)
        assert r.valid and r.n == 0 and r.rho[0] == 0.0
        p0 = O.tempered_softmax(Lt[0], T)[0]
        assert r.resid_mass == pytest.approx(1.0, rel=1e-14)
        assert r.tokens == [O.inverse_cdf(p0, u[gamma])[0]]


def test_residual_mass_is_one_minus_alpha():
    g = np.random.default_rng(5)
    V, gamma, T = 25, 2, 0.9
    hits = 0
    for _ in range(200):
        Lt = _random_rows(g, gamma + 1, V)
        Ld = Lt[:gamma] + g.normal(0, 1.0, size=(gamma, V))
        x = g.integers(0, V, size=gamma)
        u = g.integers(0, 1 << 24, size=gamma + 1) * 2.0 ** -24
        r = O.verify_sample_sequence(Lt, Ld, x, u, T)
        if r.n < gamma:
            p = O.tempered_softmax(Lt[r.n], T)[0]
            q = O.tempered_softmax(Ld[r.n], T)[0]
            assert r.resid_mass == pytest.approx(1.0 - O.alpha(p, q), abs=1e-13)
            hits += 1
    assert hits > 20


def test_zero_temperature_limit_equals_chain_tree():
    """As T -> 0 both models become one-hot: rho_i is 1 when x_i is the target's
    top token and ~0 otherwise, and the corrected token is the target's top token.
    That is the greedy tree rule on a chain, so the two oracles must agree."""
    g = np.random.default_rng(21)
    V, gamma = 12, 5
    for trial in range(60):
        # well separated logits: distinct integers times 2
        Lt = np.stack([g.permutation(V) * 2.0 for _ in range(gamma + 1)])
        Ld = np.stack([g.permutation(V) * 2.0 for _ in range(gamma)])
        # make a random-length prefix of the drafts agree with the target
        agree = int(g.integers(0, gamma + 1))
        for i in range(agree):
            Ld[i] = Lt[i]
        x = [int(np.argmax(Ld[i])) for i in range(gamma)]  # what a T -> 0 draft emits
        u = g.integers(0, 1 << 24, size=gamma + 1) * 2.0 ** -24
        u[:gamma] = np.minimum(u[:gamma], 0.999)
        r = O.verify_sample_sequence(Lt, Ld, x, u, 1e-3)
        parents = [-1] + list(range(gamma))
        tokens = [0] + x
        t = O.verify_tree_sequence(Lt, parents, tokens)
        assert r.valid and t.valid
        assert r.n == t.accept_len, trial
        assert r.tokens == x[: r.n] + [t.bonus]
