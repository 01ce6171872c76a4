"""Statistical pins of the sampling oracle on config-1 style inputs.

Expected accepted length: with i.i.d. positions (the same p and q at every
position) each draft is accepted independently with probability
alpha = sum min(p, q), so n is a truncated geometric variable and
E[n + 1] = (1 - alpha^(gamma+1)) / (1 - alpha). The pages tie the speedup to
this count ("Fast Inference from Transformers via Speculative Decoding", Pith
review: "What would settle it", "Referee Report" second minor comment).
Thresholds are fixed before running; seeds are fixed and never changed to pass.
"""
import numpy as np
import scipy.stats

import synth
from oracle import spec_verify_oracle as O


def _run(inp):
    return O.verify_sample_batch(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.temperature,
                                 "f32", "f32", shared_logits=True)


def test_expected_accepted_length_iid():
    inp = synth.make_sample_inputs(1, seed=3, trials=20000, iid=True)
    res = _run(inp)
    T = float(inp.temperature[0])
    p = O.tempered_softmax(O.widen(inp.target[0, 0], "f32"), T)[0]
    q = O.tempered_softmax(O.widen(inp.draft[0, 0], "f32"), T)[0]
    a = O.alpha(p, q)
    G = inp.gamma
    ns = np.array([r.n for r in res])
    assert all(r.valid for r in res)
    mean_closed = (1 - a ** (G + 1)) / (1 - a)
    pmf = np.array([a ** k * (1 - a) for k in range(G)] + [a ** G])
    k = np.arange(G + 1)
    var = float(np.sum(pmf * (k + 1) ** 2) - np.sum(pmf * (k + 1)) ** 2)
    tol = 4 * np.sqrt(var / len(ns))
    assert abs(np.mean(ns + 1) - mean_closed) < tol, (np.mean(ns + 1), mean_closed, tol)
    # and the whole law of n: P(n = k) = alpha^k (1 - alpha), P(n = gamma) = alpha^gamma
    counts = np.bincount(ns, minlength=G + 1)
    chi = scipy.stats.chisquare(counts, pmf * len(ns))
    assert chi.pvalue > 0.01


def test_first_emitted_token_follows_p0():
    inp = synth.make_sample_inputs(1, seed=4, trials=20000)
    res = _run(inp)
    T = float(inp.temperature[0])
    p0 = O.tempered_softmax(O.widen(inp.target[0, 0], "f32"), T)[0]
    first = np.array([r.tokens[0] for r in res])
    counts = np.bincount(first, minlength=p0.size).astype(float)
    exp = p0 * len(first)
    # pool bins with expected count < 5 into one
    small = exp < 5
    obs = np.concatenate([counts[~small], [counts[small].sum()]]) if small.any() else counts
    ex = np.concatenate([exp[~small], [exp[small].sum()]]) if small.any() else exp
    assert scipy.stats.chisquare(obs, ex).pvalue > 0.01
