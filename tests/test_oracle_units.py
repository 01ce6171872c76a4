"""Pins of the oracle's building blocks against library routines and hand cases."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import spec_verify_oracle as O


def _rows(seed, n=20, V=50, mask=True):
    g = np.random.default_rng(seed)
    rows = g.normal(0, 3, size=(n, V))
    if mask:
        m = g.random((n, V)) < 0.2
        m[:, 0] = False
        rows[m] = -np.inf
    return rows


@pytest.mark.parametrize("T", [0.05, 0.7, 1.0, 10.0])
def test_softmax_matches_scipy(T):
    for row in _rows(1):
        p, m, s = O.tempered_softmax(row, T)
        ref = scipy.special.softmax(row / T)
        np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)
        assert abs(p.sum() - 1.0) < 1e-14
        assert m == row.max()
        # log-probabilities agree with scipy's log_softmax (log-sum-exp route)
        lref = scipy.special.log_softmax(row / T)
        for v in np.flatnonzero(np.isfinite(row))[:5]:
            assert abs(O.log_prob(row, T, m, s, v) - lref[v]) < 1e-12 * max(1.0, abs(lref[v]))


def test_inverse_cdf_hand_cases():
    r = np.array([0.25, 0.25, 0.5])  # exact binary fractions: C = [0.25, 0.5, 1.0]
    assert O.inverse_cdf(r, 0.0)[0] == 0
    assert O.inverse_cdf(r, 0.25)[0] == 1  # intervals are half-open [C_{k-1}, C_k)
    assert O.inverse_cdf(r, 0.4999)[0] == 1
    assert O.inverse_cdf(r, 0.5)[0] == 2
    assert O.inverse_cdf(r, 1 - 2 ** -24)[0] == 2
    z = np.array([0.0, 0.0, 0.5, 0.0, 0.5, 0.0])
    assert O.inverse_cdf(z, 0.0)[0] == 2  # zero-mass tokens are never drawn
    assert O.inverse_cdf(z, 0.5)[0] == 4
    assert O.inverse_cdf(z, 1 - 2 ** -24)[0] == 4


def test_inverse_cdf_brute_force():
    g = np.random.default_rng(7)
    for _ in range(300):
        V = int(g.integers(1, 12))
        r = g.random(V) * (g.random(V) < 0.6)
        if r.sum() == 0:
            r[int(g.integers(0, V))] = 0.3
        u = float(g.integers(0, 1 << 24)) * 2 ** -24
        y, C, S = O.inverse_cdf(r, u)
        # brute force: total mass, then walk the tokens in order with running sums
        total = 0.0
        for v in range(V):
            total += float(r[v])
        t = u * total
        acc = 0.0
        want = None
        for v in range(V):
            acc += r[v]
            if acc > t:
                want = v
                break
        assert y == want
        assert r[y] > 0


def test_argmax_first_special_cases():
    assert O.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert O.argmax_first(np.array([-0.0, 0.0])) == 0
    assert O.argmax_first(np.array([0.0, -0.0])) == 0
    assert O.argmax_first(np.array([-np.inf, -np.inf, -np.inf])) == 0
    assert O.argmax_first(np.array([-np.inf, -5.0, -np.inf])) == 1
    g = np.random.default_rng(3)
    for _ in range(200):
        row = g.integers(-3, 4, size=int(g.integers(1, 40))).astype(np.float64)
        mx = max(row)
        assert O.argmax_first(row) == next(i for i, v in enumerate(row) if v == mx)


def test_alpha_special_cases():
    p = np.array([0.2, 0.3, 0.5])
    assert O.alpha(p, p) == pytest.approx(1.0, abs=1e-15)
    assert O.alpha(np.array([1.0, 0, 0]), np.array([0, 0.5, 0.5])) == 0.0
    # two-point closed form: alpha = 1 - |p0 - q0|
    for a, b in [(0.1, 0.7), (0.5, 0.5), (0.9, 0.2)]:
        assert O.alpha(np.array([a, 1 - a]), np.array([b, 1 - b])) == pytest.approx(1 - abs(a - b), abs=1e-15)


def test_widen_bf16_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x8000, 0x0000, 0x3F81, 0x0001], dtype=np.uint16)
    w = O.widen(bits, "bf16")
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == np.inf and w[3] == -np.inf
    assert w[4] == 0.0 and math.copysign(1, w[4]) == -1.0 and w[5] == 0.0
    assert w[6] == 1.0 + 2 ** -7
    assert w[7] == 2.0 ** -133  # smallest bf16 subnormal
    assert np.isnan(O.widen(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")).all()


def test_temperature_and_row_validity():
    assert O.temperature_is_valid(1.0) and O.temperature_is_valid(1e-30)
    assert not O.temperature_is_valid(0.0) and not O.temperature_is_valid(-1.0)
    assert not O.temperature_is_valid(float("inf")) and not O.temperature_is_valid(float("nan"))
    assert not O.temperature_is_valid(1e-40)  # subnormal
    assert O.row_is_valid(np.array([-np.inf, 0.0]))
    assert not O.row_is_valid(np.array([-np.inf, -np.inf]))
    assert not O.row_is_valid(np.array([0.0, np.nan]))
    assert not O.row_is_valid(np.array([0.0, np.inf]))


def test_residual_and_its_fallback():
    p = np.array([0.5, 0.25, 0.25])
    q = np.array([0.25, 0.25, 0.5])
    r, fb = O.residual(p, q)
    assert not fb and list(r) == [0.25, 0.0, 0.0]
    # p <= q everywhere (equal up to one rounding step): nothing left to redraw from
    q2 = np.array([0.5, 0.25, 0.25 + 2 ** -52])
    r2, fb2 = O.residual(p, q2)
    assert fb2 and np.array_equal(r2, p)
