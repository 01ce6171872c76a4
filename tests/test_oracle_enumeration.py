"""Exact output law of the sampling oracle on tiny vocabularies.

The pages' central claim is that speculative sampling changes nothing about
the output: the emitted tokens are exact samples of the target model
("Fast Inference from Transformers via Speculative Decoding", Pith review:
abstract, "Core claim", "Circularity Check"). With position-dependent but
context-free target rows p_0..p_gamma, plain autoregressive sampling emits
z_k ~ p_k independently, so the law of the emitted prefix, completed with
independent draws from the remaining rows, must be prod_k p_k(z_k).

The oracle is a deterministic function of (drafts x, uniforms u). For every
draft tuple (weight prod q_i(x_i)) the unit cube of uniforms splits into cells
on which the output is constant: accept cells [0, min(1, rho_i)), reject cells
[min(1, rho_n), 1), draw cells [C_{k-1}/S, C_k/S). The test computes those
cells itself (scipy softmax), calls the oracle once at each cell's midpoint,
weights the result by the cell's volume and compares the accumulated law with
prod_k p_k to 1e-12. A dropped term, a swapped p/q, a wrong uniform or a wrong
residual all change the law.
"""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import spec_verify_oracle as O


def _law_via_oracle(Lt, Ld, T):
    gamma, V = Ld.shape
    P = [scipy.special.softmax(Lt[k] / T) for k in range(gamma + 1)]
    Q = [scipy.special.softmax(Ld[i] / T) for i in range(gamma)]
    law = {}
    for x in itertools.product(range(V), repeat=gamma):
        wx = float(np.prod([Q[i][x[i]] for i in range(gamma)]))
        if wx == 0.0:
            continue
        acc = [min(1.0, P[i][x[i]] / Q[i][x[i]]) for i in range(gamma)]
        for n in range(gamma + 1):
            w = wx * float(np.prod(acc[:n]))
            u = [0.5] * (gamma + 1)
            for i in range(n):
                u[i] = acc[i] / 2
            if n < gamma:
                w *= 1.0 - acc[n]
                u[n] = (acc[n] + 1.0) / 2
                r = np.maximum(0.0, P[n] - Q[n])
            else:
                r = P[gamma]
            if w == 0.0 or r.sum() == 0.0:
                continue
            C = np.cumsum(r)
            S = C[-1]
            lo = 0.0
            for k in range(V):
                if r[k] == 0.0:
                    continue
                hi = C[k] / S
                u[gamma] = (lo + hi) / 2
                res = O.verify_sample_sequence(Lt, Ld, x, u, T)
                assert res.valid
                assert res.n == n and res.y == k, (x, n, k, res.n, res.y)
                z = tuple(res.tokens)
                law[z] = law.get(z, 0.0) + w * (hi - lo)
                lo = hi
    # complete each emitted prefix with independent draws from the remaining rows
    full = {}
    for z, w in law.items():
        rest = range(len(z), gamma + 1)
        for tail in itertools.product(range(V), repeat=len(rest)):
            wt = w * float(np.prod([P[k][t] for k, t in zip(rest, tail)]))
            key = z + tail
            full[key] = full.get(key, 0.0) + wt
    return full, P


@pytest.mark.parametrize("V,gamma", [(2, 1), (2, 3), (3, 1), (3, 2), (4, 2), (3, 3)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_law_equals_target(V, gamma, seed):
    g = np.random.default_rng(100 * V + 10 * gamma + seed)
    T = [1.0, 0.6, 1.7][seed]
    Lt = g.normal(0, 1.5, size=(gamma + 1, V))
    Ld = g.normal(0, 1.5, size=(gamma, V))
    if seed == 1 and V > 2:  # masks: a token the target never emits, one the draft never proposes
        Lt[0, 0] = -np.inf
        Ld[gamma - 1, V - 1] = -np.inf
    full, P = _law_via_oracle(Lt, Ld, T)
    for z in itertools.product(range(V), repeat=gamma + 1):
        want = float(np.prod([P[k][z[k]] for k in range(gamma + 1)]))
        assert abs(full.get(z, 0.0) - want) < 1e-12, (z, full.get(z, 0.0), want)
    assert abs(sum(full.values()) - 1.0) < 1e-12
