"""Pins of the oracle's end-to-end loop on a Markov-chain model pair: the
emitted stream has the target chain's law (chi-square of transition counts,
over many calls), and the expected tokens per call match their closed forms and
a Monte-Carlo run of the loop."""
import numpy as np
from scipy import stats

import synth
from oracle import spec_verify_oracle as O


def _tables(V, seed, noise=0.8):
    t = synth.make_markov_tables(V, "f32", seed=seed, noise_sd=noise)
    return t.target.astype(np.float64), t.draft.astype(np.float64)


def test_expected_tokens_closed_forms():
    Lt, Ld = _tables(6, 1)
    P, Q = O.markov_transitions(Lt, 0.9), O.markov_transitions(Ld, 0.9)
    e1 = O.expected_tokens_per_call(P, Q, 1)
    assert np.allclose(e1, 1 + np.minimum(P, Q).sum(axis=1), rtol=0, atol=1e-14)
    assert np.allclose(O.expected_tokens_per_call(P, P, 5), 6.0, rtol=0, atol=1e-12)
    # state-independent overlap: a chain whose rows are all the same reduces to the i.i.d. closed form
    Pr = np.tile(P[0], (6, 1))
    Qr = np.tile(Q[0], (6, 1))
    a = O.alpha(P[0], Q[0])
    assert np.allclose(O.expected_tokens_per_call(Pr, Qr, 4), (1 - a ** 5) / (1 - a), rtol=1e-12)


def test_loop_stream_law_and_tokens_per_call():
    """20000 calls on V = 5, gamma = 3: the transition counts of the emitted
    stream follow P (chi-square per source token, pooled), and the mean tokens
    per call from each start token match expected_tokens_per_call within 4
    standard errors."""
    V, G, T, K, chains = 5, 3, 1.0, 1000, 20
    Lt, Ld = _tables(V, 2, noise=1.0)
    P, Q = O.markov_transitions(Lt, T), O.markov_transitions(Ld, T)
    E = O.expected_tokens_per_call(P, Q, G)
    g = np.random.default_rng(3)
    counts = np.zeros((V, V))
    per_start = [[] for _ in range(V)]
    for c in range(chains):
        s = c % V
        res = O.markov_loop(Lt, Ld, T, s, g.random((K, G)), g.random((K, G + 1)))
        assert len(res) == K
        prev = s
        for n, emitted in res:
            per_start[prev].append(n + 1)
            for tok in emitted:
                counts[prev, tok] += 1
                prev = tok
    chi, dof = 0.0, 0
    for s in range(V):
        exp = P[s] * counts[s].sum()
        chi += ((counts[s] - exp) ** 2 / exp).sum()
        dof += V - 1
    p = stats.chi2.sf(chi, dof)
    assert p > 1e-3, (chi, dof, p)
    for s in range(V):
        x = np.asarray(per_start[s], float)
        assert abs(x.mean() - E[s]) < 4 * x.std() / np.sqrt(len(x)) + 1e-9, (s, x.mean(), E[s])
