"""Plain fp64 CPU oracle for the speculative verify step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the package entry
point and the CPU-baseline leg of the benchmark use it. It shares no code with
the HIP path (no kernels, headers, helpers, tables or pre/post-processing); it
is numpy in float64 throughout, one sequence at a time, with no fusion,
chunking or online rescaling.

What it computes, and where the pages define it
------------------------------------------------
Sources are the text of four web pages:
  [SD]     "Fast Inference from Transformers via Speculative Decoding" --
           Pith review page (pith.science, arXiv 2211.17192).
  [SD-cc]  The CoChat page on the same paper (app.cochat.ai).
  [SS]     The "speculative sampling" summary page (ar.omco.ai, arXiv 2302.01318).
  [Falcon] "Falcon: Faster and Parallel Inference of Large Language Models
           through Enhanced Semi-Autoregressive Drafting and Custom-Designed
           Decoding Tree" -- Pith review page (pith.science, arXiv 2412.12639).

Sampling verify (one sequence): [SD] "The pith" and "What carries the
argument" describe one parallel target pass scoring the gamma drafted tokens
and keeping the longest accepted prefix; [SD] "Desk Editor's Note" and
"Referee Report" (Summary, Significance) name the correction a rejection
sampling step whose acceptance probability comes from the target conditional;
[SD] abstract, "Core claim" and "Circularity Check" fix the invariant: the
emitted tokens are exact samples of the target distribution. The accept
probability min(1, p(x)/q(x)) and the residual max(0, p - q) are the unique
choice that makes that invariant hold for drafts x ~ q (derivation in
``verify_sample_sequence``). Temperature is applied to both models' logits.

Greedy tree verify (one sequence): [Falcon] "What carries the argument" --
the drafter proposes a tree of candidate branches that the target checks in
one parallel pass; [Falcon] "Assumptions & free parameters" and Figure 4
(temperature 0): greedy output must equal vanilla autoregressive decoding, so
a node is accepted exactly when its token is the target's argmax after its
parent and every ancestor is accepted.

Readings where the pages are silent (each also listed in the design notes):
  * accept iff u < rho (strict); uniforms live in [0, 1);
  * u[i] drives the accept test of position i, u[gamma] drives the single final
    draw (residual after a rejection, bonus row after full acceptance);
  * inverse CDF in token-id order: y = smallest v with C[v] > u * S on the
    unnormalised residual r, C = running sum, S = C[V-1];
  * S == 0 after a rejection (possible only if p_n == q_n) draws from p_n and
    is flagged;
  * argmax ties go to the lowest index, -0 == +0; NaN or +inf in a consumed row
    makes the sequence invalid; -inf is a mask;
  * the deepest accepted tree node wins, ties to the lowest node index.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FLT_MIN_NORMAL = 2.0 ** -126
FLT_MAX = float(np.finfo(np.float32).max)


# ----------------------------------------------------------------------------
# input widening (oracle's own; bf16 is the upper half of an IEEE binary32)
# ----------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored logits: 'bf16' (uint16 bit patterns) or 'f32'."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------
def row_is_valid(row: np.ndarray) -> bool:
    """A logit row is usable iff it has no NaN, no +inf and at least one finite value."""
    if np.isnan(row).any() or (row == np.inf).any():
        return False
    return bool((row > -np.inf).any())


def temperature_is_valid(T: float) -> bool:
    """Temperature must be a finite, normal, positive binary32 value."""
    return bool(np.isfinite(T) and FLT_MIN_NORMAL <= T <= FLT_MAX)


def tempered_softmax(row: np.ndarray, T: float):
    """p_v = exp((L_v - m)/T) / sum_w exp((L_w - m)/T), m = max_v L_v.

    Returns (p, m, s) with s the sum of the shifted exponentials.
    -inf logits give p_v = 0.
    """
    m = np.max(row)
    e = np.exp((row - m) / T)
    s = np.sum(e)
    return e / s, m, s


def log_prob(row: np.ndarray, T: float, m: float, s: float, v: int) -> float:
    """log p_v = (L_v - m)/T - log s  (same quantity as log of tempered_softmax)."""
    return (row[v] - m) / T - np.log(s)


def alpha(p: np.ndarray, q: np.ndarray) -> float:
    """Draft/target overlap alpha = sum_v min(p_v, q_v): the probability that a
    draft x ~ q is accepted. ([SD] "Referee Report", second minor comment, and
    "What would settle it": the expected accepted count rests on it.)"""
    return float(np.sum(np.minimum(p, q)))


def inverse_cdf(r: np.ndarray, u: float):
    """Smallest index y with C[y] > u * S, C = cumulative sum of r in index order.

    ``r`` is non-negative with S = C[-1] > 0 and 0 <= u < 1, so u*S < S and such
    a y exists with r[y] > 0. Returns (y, C, S).
    """
    C = np.cumsum(r)
    S = C[-1]
    t = u * S
    y = int(np.searchsorted(C, t, side="right"))
    return y, C, S


def residual(p: np.ndarray, q: np.ndarray):
    """r = max(0, p - q) element-wise, the distribution a rejected position is
    redrawn from (up to normalisation). If it is identically zero -- reachable
    only when p == q up to rounding, where a rejection has probability zero --
    fall back to p and flag it. Returns (r, fell_back)."""
    r = np.maximum(0.0, p - q)
    if np.sum(r) == 0.0:
        return p.copy(), True
    return r, False


def argmax_first(row: np.ndarray) -> int:
    """Index of the largest value, lowest index on ties (float compare: -0 == +0)."""
    return int(np.argmax(row))


# ----------------------------------------------------------------------------
# sampling verify
# ----------------------------------------------------------------------------
@dataclass
class SampleResult:
    valid: bool
    n: int = -1  # accepted drafts, 0..gamma; -1 invalid
    tokens: list = field(default_factory=list)  # x_0..x_{n-1}, y
    y: int = -1
    rho: np.ndarray | None = None  # [gamma] p_i(x_i)/q_i(x_i); NaN where not computed
    p_x: np.ndarray | None = None  # [gamma]
    q_x: np.ndarray | None = None  # [gamma]
    alphas: np.ndarray | None = None  # [gamma] sum min(p_i, q_i) (computed rows only)
    resid_mass: float = float("nan")  # S / normaliser: 1 - alpha_n after a rejection, 1 for the bonus
    draw_row: int = -1  # which row the final draw used (n)
    bonus: bool = False
    fallback: bool = False  # S == 0 after a rejection: drew from p_n instead
    cdf: np.ndarray | None = None  # normalised C/S of the drawn distribution (if kept)
    consumed: int = 0  # number of accept tests evaluated


def verify_sample_sequence(Lt: np.ndarray, Ld: np.ndarray, x, u, T: float, keep_cdf: bool = False,
                           with_alpha: bool = False) -> SampleResult:
    """One sequence of speculative sampling verification, in float64.

    Lt: [gamma+1][V] target logits; row i is the target's next-token logits
        after the prefix and drafts x_0..x_{i-1}; row gamma is the bonus row.
    Ld: [gamma][V] draft logits; row i is what x_i was drawn from.
    x : [gamma] draft tokens. u: [gamma+1] uniforms in [0, 1). T: temperature.

    Steps, in the order the method takes them:
      1. p_i = softmax(Lt_i / T), q_i = softmax(Ld_i / T).
      2. For i = 0, 1, ...: rho_i = p_i(x_i)/q_i(x_i); accept x_i iff u_i < rho_i
         (accept probability min(1, rho_i)); stop at the first rejection n
         (the longest accepted prefix, [SD] "The pith"). n = gamma if none.
      3. After a rejection at n: draw y from r = max(0, p_n - q_n) renormalised;
         after full acceptance: draw y from p_gamma (the bonus row).
         Why r: with x ~ q, P(emit z by acceptance) = min(p(z), q(z)) and
         P(reject) = 1 - sum_z min(p, q); the emitted token has law p only if
         the rejected branch carries mass p(z) - min(p(z), q(z)) = max(0, p(z) - q(z)).
      4. y = inverse CDF of r in token order at u_gamma.
    Rows, tokens and uniforms that the steps above never reach are not checked.
    """
    Lt = np.asarray(Lt, dtype=np.float64)
    Ld = np.asarray(Ld, dtype=np.float64)
    gamma = Ld.shape[0]
    V = Lt.shape[1]
    x = [int(t) for t in x]
    u = np.asarray(u, dtype=np.float64)
    res = SampleResult(valid=False, rho=np.full(gamma, np.nan), p_x=np.full(gamma, np.nan),
                       q_x=np.full(gamma, np.nan), alphas=np.full(gamma, np.nan))
    if not temperature_is_valid(float(T)):
        return res
    T = float(T)

    def u_ok(v):
        return bool(0.0 <= v < 1.0)

    n = gamma
    p_rows = {}
    q_rows = {}
    for i in range(gamma):
        if not (row_is_valid(Lt[i]) and row_is_valid(Ld[i])):
            return res
        if not (0 <= x[i] < V) or Ld[i][x[i]] == -np.inf or not u_ok(u[i]):
            return res
        p, mp, sp = tempered_softmax(Lt[i], T)
        q, mq, sq = tempered_softmax(Ld[i], T)
        p_rows[i], q_rows[i] = p, q
        lp = log_prob(Lt[i], T, mp, sp, x[i])
        lq = log_prob(Ld[i], T, mq, sq, x[i])
        res.rho[i] = np.exp(lp - lq)
        res.p_x[i] = np.exp(lp)
        res.q_x[i] = np.exp(lq)
        if with_alpha:
            res.alphas[i] = alpha(p, q)
        res.consumed = i + 1
        if not (u[i] < res.rho[i]):
            n = i
            break
    if not u_ok(u[gamma]):
        return res
    if n == gamma:
        if not row_is_valid(Lt[gamma]):
            return res
        r, _, _ = tempered_softmax(Lt[gamma], T)
        res.bonus = True
    else:
        r, res.fallback = residual(p_rows[n], q_rows[n])
    y, C, S = inverse_cdf(r, float(u[gamma]))
    res.valid = True
    res.n = n
    res.y = y
    res.tokens = x[:n] + [y]
    res.draw_row = n
    res.resid_mass = float(S)  # r is built from normalised p, q: S is already a probability mass
    if keep_cdf:
        res.cdf = C / S
    return res


def verify_sample_batch(Lt_all, Ld_all, tokens, uniforms, temps, t_dtype="f32", d_dtype="f32",
                        seqs=None, shared_logits=False, **kw):
    """Apply ``verify_sample_sequence`` to each listed sequence (default: all)."""
    B = tokens.shape[0]
    seqs = range(B) if seqs is None else seqs
    out = []
    for b in seqs:
        lb = 0 if shared_logits else b
        Lt = widen(Lt_all[lb], t_dtype)
        Ld = widen(Ld_all[lb], d_dtype)
        out.append(verify_sample_sequence(Lt, Ld, tokens[b], uniforms[b], float(temps[b]), **kw))
    return out


# ----------------------------------------------------------------------------
# greedy tree verify
# ----------------------------------------------------------------------------
@dataclass
class DraftResult:
    valid: bool
    y: int = -1
    q_y: float = float("nan")
    cdf: np.ndarray | None = None


def draft_sample_row(L: np.ndarray, T: float, u: float, keep_cdf: bool = False) -> DraftResult:
    """The draft-side step that produces the inputs of the verify: x ~ q with
    q = softmax(L / T) ([SD] "The pith" and the abstract: the fast
    approximation model proposes the speculative tokens by sampling from its
    own distribution). Drawn by inverse CDF in token-id order at u, the same
    rule as the verify's final draw. Invalid (y = -1) for an unusable
    temperature, a uniform outside [0, 1) or a row with NaN, +inf or no finite
    value."""
    if not temperature_is_valid(T) or not (0.0 <= u < 1.0) or not row_is_valid(L):
        return DraftResult(False)
    q, _, _ = tempered_softmax(L, T)
    y, C, S = inverse_cdf(q, u)
    return DraftResult(True, y, float(q[y]), C / S if keep_cdf else None)


@dataclass
class TreeResult:
    valid: bool
    accept_len: int = -1
    path: list = field(default_factory=list)  # node ids root-first, 0..d
    bonus: int = -1
    argmax: np.ndarray | None = None  # [N] per-node argmax; -1 for an unusable row


def tree_is_valid(parents, tokens, V: int) -> bool:
    """Parent array: parents[0] = -1 and 0 <= parents[j] < j; node tokens in [0, V) for j >= 1."""
    N = len(parents)
    if N < 1 or int(parents[0]) != -1:
        return False
    for j in range(1, N):
        if not (0 <= int(parents[j]) < j):
            return False
        if not (0 <= int(tokens[j]) < V):
            return False
    return True


def row_has_nan_or_posinf(row: np.ndarray) -> bool:
    return bool(np.isnan(row).any() or (row == np.inf).any())


def verify_tree_sequence(L: np.ndarray, parents, tokens) -> TreeResult:
    """Greedy verification of one draft tree.

    L: [N][V] target logits, row j = next-token logits after node j.
    1. g_j = argmax_v L[j][v] (lowest index on ties).
    2. acc[0] = true; for j = 1..N-1 in index order:
       acc[j] = acc[parents[j]] and tokens[j] == g[parents[j]].
    3. depth[j] = depth[parents[j]] + 1; d = accepted node of largest depth,
       lowest index on ties.
    4. path = root .. d; accepted length = depth[d]; bonus = g[d].
    """
    L = np.asarray(L, dtype=np.float64)
    N, V = L.shape
    g = np.full(N, -1, dtype=np.int64)
    bad_row = False
    for j in range(N):
        if row_has_nan_or_posinf(L[j]):
            bad_row = True
        else:
            g[j] = argmax_first(L[j])
    res = TreeResult(valid=False, argmax=g)
    if bad_row or not tree_is_valid(parents, tokens, V):
        return res
    acc = [False] * N
    depth = [0] * N
    acc[0] = True
    for j in range(1, N):
        pj = int(parents[j])
        depth[j] = depth[pj] + 1
        acc[j] = acc[pj] and int(tokens[j]) == int(g[pj])
    d = 0
    for j in range(N):
        if acc[j] and depth[j] > depth[d]:
            d = j
    path = []
    k = d
    while k != -1:
        path.append(k)
        k = int(parents[k])
    path.reverse()
    res.valid = True
    res.accept_len = depth[d]
    res.path = path
    res.bonus = int(g[d])
    return res


def greedy_walk(L: np.ndarray, parents, tokens) -> TreeResult:
    """Second, independent definition: greedy autoregressive decoding confined to the tree.

    Start at the root; the target's greedy next token after the current node is
    g[cur]; move to a child carrying that token (if several, the one whose
    matching descendants reach deepest, lowest index on ties) and repeat; stop
    when no child matches. The emitted tokens are those of the visited nodes
    followed by g[last]: what vanilla greedy decoding would have produced
    ([Falcon] "Assumptions & free parameters").
    """
    L = np.asarray(L, dtype=np.float64)
    N, V = L.shape
    g = [argmax_first(L[j]) for j in range(N)]
    kids = [[] for _ in range(N)]
    for j in range(1, N):
        kids[int(parents[j])].append(j)

    def reach(c):  # how many more matching steps can be taken below node c
        best = 0
        for k in kids[c]:
            if int(tokens[k]) == g[c]:
                best = max(best, 1 + reach(k))
        return best

    cur = 0
    path = [0]
    while True:
        match = [k for k in kids[cur] if int(tokens[k]) == g[cur]]
        if not match:
            break
        depths = [reach(k) for k in match]
        top = max(depths)
        cur = min(k for k, dd in zip(match, depths) if dd == top)
        path.append(cur)
    return TreeResult(valid=True, accept_len=len(path) - 1, path=path, bonus=g[cur],
                      argmax=np.array(g, dtype=np.int64))


def verify_tree_batch(logits, parents, tokens, dtype="bf16", seqs=None):
    B = parents.shape[0]
    seqs = range(B) if seqs is None else seqs
    return [verify_tree_sequence(widen(logits[b], dtype), parents[b], tokens[b]) for b in seqs]


# ----------------------------------------------------------------------------
# end-to-end loop on a Markov-chain model pair
# ----------------------------------------------------------------------------
def markov_transitions(table: np.ndarray, T: float) -> np.ndarray:
    """P[s] = softmax(table[s] / T): the tempered next-token law after token s
    of a first-order Markov 'model' whose logits after s are table[s]."""
    return np.stack([tempered_softmax(table[s], T)[0] for s in range(table.shape[0])])


def expected_tokens_per_call(P: np.ndarray, Q: np.ndarray, gamma: int) -> np.ndarray:
    """E[n + 1 | s0] for every start token s0: tokens emitted by one verify call
    (accepted drafts plus the corrected or bonus token) when the draft chain
    has law Q and the target chain law P.

    A draft x ~ q is accepted with probability min(1, p(x)/q(x)), so a position
    after token s emits an accepted token v with probability min(P[s, v],
    Q[s, v]) ([SD] "Referee Report", second minor comment: the accepted count
    rests on this overlap). With M = min(P, Q) element-wise, the probability
    that the first k drafts are all accepted, from s0, is (M^k 1)[s0]; the call
    emits n + 1 tokens and E[n + 1] = sum_{k=0..gamma} (M^k 1)[s0]. For i.i.d.
    positions this is the closed form (1 - alpha^(gamma+1)) / (1 - alpha)."""
    M = np.minimum(P, Q)
    v = np.ones(P.shape[0])
    total = v.copy()
    for _ in range(gamma):
        v = M @ v
        total += v
    return total


def markov_loop(Lt_table: np.ndarray, Ld_table: np.ndarray, T: float, state0: int, u_draft: np.ndarray,
                u_verify: np.ndarray):
    """Speculative decoding of one chain for len(u_draft) iterations ([SD]
    "The pith": the draft proposes gamma tokens from its own law, the target
    scores them in one pass, the longest accepted prefix and one corrected or
    bonus token are kept). Iteration k draws x_i ~ q(. | previous token) with
    draft_sample_row at u_draft[k][i], then verifies with verify_sample_sequence
    on target rows Lt_table[s], Lt_table[x_0], ..., Lt_table[x_{gamma-1}] and
    draft rows Ld_table[s], Ld_table[x_0], ..., Ld_table[x_{gamma-2}] at
    u_verify[k]. Returns a list of (n, emitted tokens) per iteration; stops at
    an invalid step."""
    out = []
    s = int(state0)
    K, gamma = u_draft.shape
    for k in range(K):
        prev = s
        x = []
        for i in range(gamma):
            r = draft_sample_row(Ld_table[prev], T, float(u_draft[k, i]))
            if not r.valid:
                return out
            x.append(r.y)
            prev = r.y
        rows_t = Lt_table[[s] + x]
        rows_d = Ld_table[[s] + x[:-1]]
        res = verify_sample_sequence(rows_t, rows_d, x, u_verify[k].astype(np.float64), T)
        if not res.valid:
            return out
        emitted = list(x[: res.n]) + [res.y]
        out.append((res.n, emitted))
        s = emitted[-1]
    return out


# ----------------------------------------------------------------------------
# draft-tree attention masks
# ----------------------------------------------------------------------------
def parents_valid(parents) -> bool:
    """parents[0] = -1 and 0 <= parents[j] < j for j >= 1."""
    N = len(parents)
    if N == 0 or int(parents[0]) != -1:
        return False
    return all(0 <= int(parents[j]) < j for j in range(1, N))


def tree_masks(parents, blocks=None):
    """Attention masks of one draft tree ([Falcon] "What carries the
    argument": the target checks every branch of the tree in one pass, so a
    node sees exactly its own path to the root; the drafter's relaxed causal
    mask also lets the tokens of one block see each other).

    Returns (mask, relaxed, depth): mask[i][j] = 1 iff j == i or j is an
    ancestor of i; relaxed = mask or (blocks[i] >= 0 and blocks[i] ==
    blocks[j]) (None without blocks); depth[i] = number of parent steps to the
    root. An invalid parent array gives all-zero masks and depth -1."""
    N = len(parents)
    mask = np.zeros((N, N), dtype=np.uint8)
    depth = np.full(N, -1, dtype=np.int32)
    relaxed = None if blocks is None else np.zeros((N, N), dtype=np.uint8)
    if not parents_valid(parents):
        return mask, relaxed, depth
    for i in range(N):
        a, d = i, 0
        while a >= 0:
            mask[i, a] = 1
            a = int(parents[a])
            d += 1
        depth[i] = d - 1
    if blocks is not None:
        for i in range(N):
            for j in range(N):
                relaxed[i, j] = 1 if mask[i, j] or (blocks[i] >= 0 and blocks[i] == blocks[j]) else 0
    return mask, relaxed, depth
