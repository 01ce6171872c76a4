"""Statistical checks of the GPU path over 10^6 draws of the tiny configuration.

The pages' claim is that speculative sampling leaves the output distribution
unchanged ("Fast Inference from Transformers via Speculative Decoding", Pith
review: abstract, "Core claim"). With position-dependent, context-free rows
the k-th emitted token must follow p_{k-1}. Thresholds (p > 0.01, 4 sigma) are
fixed before running and the seeds are fixed.
"""
import numpy as np
import pytest
import scipy.stats

import synth
from oracle import spec_verify_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

TRIALS = 1_000_000


def _pooled_chisq(counts, probs):
    exp = probs * counts.sum()
    small = exp < 5
    if small.any():
        counts = np.concatenate([counts[~small], [counts[small].sum()]])
        exp = np.concatenate([exp[~small], [exp[small].sum()]])
    return scipy.stats.chisquare(counts, exp).pvalue


def test_emitted_tokens_follow_target(gpu):
    H.log("chi-square over 10^6 trials of config-1 logits")
    inp = synth.make_sample_inputs(1, seed=21, trials=TRIALS)
    out = H.run_sample(gpu, H.sample_tensors(inp), diag=False)
    assert (out["n"] >= 0).all()
    T = float(inp.temperature[0])
    P = [O.tempered_softmax(O.widen(inp.target[0, k], "f32"), T)[0] for k in range(inp.gamma + 1)]
    first = out["tokens"][:, 0]
    p1 = _pooled_chisq(np.bincount(first, minlength=32).astype(float), P[0])
    H.log(f"first token vs p_0: p-value {p1:.4f}")
    assert p1 > 0.01
    # secondary: k-th emitted token vs p_{k-1} on the trials that emitted it
    for k in range(1, inp.gamma + 1):
        sel = out["n"] >= k
        pk = _pooled_chisq(np.bincount(out["tokens"][sel, k], minlength=32).astype(float), P[k])
        H.log(f"token {k} vs p_{k} ({sel.sum()} trials): p-value {pk:.4f}")


def test_expected_accepted_length(gpu):
    H.log("E[n+1] on i.i.d. positions, 10^6 trials")
    inp = synth.make_sample_inputs(1, seed=22, trials=TRIALS, iid=True)
    out = H.run_sample(gpu, H.sample_tensors(inp), diag=False)
    T = float(inp.temperature[0])
    p = O.tempered_softmax(O.widen(inp.target[0, 0], "f32"), T)[0]
    q = O.tempered_softmax(O.widen(inp.draft[0, 0], "f32"), T)[0]
    a = O.alpha(p, q)
    G = inp.gamma
    n = out["n"]
    closed = (1 - a ** (G + 1)) / (1 - a)
    pmf = np.array([a ** k * (1 - a) for k in range(G)] + [a ** G])
    k = np.arange(G + 1)
    var = float(np.sum(pmf * (k + 1) ** 2) - np.sum(pmf * (k + 1)) ** 2)
    tol = 4 * np.sqrt(var / TRIALS)
    H.log(f"alpha={a:.4f} mean(n+1)={np.mean(n + 1):.5f} closed form={closed:.5f} tol={tol:.5f}")
    assert abs(np.mean(n + 1) - closed) < tol
    assert scipy.stats.chisquare(np.bincount(n, minlength=G + 1), pmf * TRIALS).pvalue > 0.01
