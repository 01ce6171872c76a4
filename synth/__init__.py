"""Seeded synthetic inputs for the speculative verify step.

This module only *makes inputs*: logits, draft tokens, uniforms,
temperatures and draft trees. It holds none of the verify step's arithmetic
(no softmax, no accept test, no residual, no inverse CDF, no argmax), so the
GPU path and the fp64 oracle, which share nothing else, can both be fed from
it.

The inputs stand in for the logits that the trained models of the pages
(T5-XXL in the speculative-decoding paper; Vicuna / LLaMA2-Chat on MT-Bench,
HumanEval and GSM8K in the Falcon paper) would produce. None of those models or
datasets is used or reproduced.

Seeding: every array is drawn from
``numpy.random.Generator(PCG64(SeedSequence([seed, config, stream, b])))``,
one generator per sequence ``b`` and per stream, so a batch can be built in
parallel threads and any single sequence can be rebuilt on its own.
Streams: 0 target logits, 1 draft logits/noise, 2 structure (permutation, tree
shape, row classes, temperatures), 3 draft-token draws, 4 verify uniforms.
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

S_TARGET, S_DRAFT, S_STRUCT, S_DRAFTTOK, S_UNIFORM = 0, 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
CALIBRATION_FILE = os.path.join(_HERE, "draft_noise.json")


# --------------------------------------------------------------------------
# bf16 packing (data formatting only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN stays a quiet NaN with its sign;
    +-inf stays +-inf; values that round past the largest finite bf16 become inf,
    as IEEE rounding prescribes.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# seeding helpers
# --------------------------------------------------------------------------
def gen(seed: int, config: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config, stream, *extra])))


def uniforms_u24(g: np.random.Generator, shape) -> np.ndarray:
    """Uniforms k * 2^-24 with k uniform on [0, 2^24): exact in fp32 and fp64, < 1."""
    k = g.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_max_draw(g: np.random.Generator, logits_f64: np.ndarray, T: float) -> int:
    """Draw one token from softmax(logits / T) with the Gumbel-max construction.

    argmax_v (logits_v / T + G_v), G_v = -log(-log U_v), U_v uniform on (0, 1),
    is distributed exactly as the tempered softmax (Gumbel 1954; the
    "Gumbel-max trick"). It stands for the draft model's own sampler, the step
    *before* verification; it never forms the softmax itself. Tokens whose
    logit is -inf are never drawn.
    """
    V = logits_f64.shape[-1]
    U = g.random(V)
    U[U == 0.0] = np.nextafter(0.0, 1.0)
    z = logits_f64 / T - np.log(-np.log(U))
    return int(np.argmax(z))


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pmap(fn, items):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        return list(ex.map(fn, items))


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class SampleConfig:
    cid: int
    name: str
    B: int
    gamma: int
    V: int
    target_dtype: str  # "f32" | "bf16"
    draft_dtype: str
    target_sd: float  # N(0, sd) for the target's logit noise (sd = std deviation)
    temperature: object  # float, or ("uniform", lo, hi) per row
    alpha_goal: float | None = None
    notes: str = ""


@dataclass(frozen=True)
class TreeConfig:
    cid: int
    name: str
    B: int
    N: int
    V: int
    dtype: str
    target_sd: float
    plant_prob: float
    plant_value: float
    block: int = 2
    max_depth: int = 6
    children: tuple = (2, 3, 4)


CONFIGS = {
    1: SampleConfig(1, "tiny speculative sampling", 1, 4, 32, "f32", "f32", 2.0, 1.0,
                    notes="10^4 trials with fixed logits; draft = target + N(0, 0.5)"),
    2: SampleConfig(2, "7B-class vocab sampling", 64, 4, 32000, "bf16", "bf16", 1.5, 1.0, 0.70,
                    notes="Zipf(1.1) log-frequency bias over a seeded permutation + N(0, 1.5)"),
    3: SampleConfig(3, "large-vocab sampling", 256, 8, 128256, "bf16", "bf16", 2.0, 0.7, 0.60),
    4: TreeConfig(4, "greedy decoding tree", 32, 60, 32000, "bf16", 2.0, 0.75, 16.0),
    5: SampleConfig(5, "stress sampling", 512, 5, 256000, "bf16", "f32", 2.0, ("uniform", 0.3, 1.5), 0.70,
                    notes="10% disjoint-support rows, 10% identical rows, the rest alpha ~ 0.7"),
}

# Config 1 draft noise is given directly (N(0, 0.5)); the others are calibrated
# (draft_noise.json, written by oracle/calibrate_draft_noise.py).
CONFIG1_DRAFT_SD = 0.5
# Config 5 "disjoint" rows: the draft keeps only tokens whose target logit is
# below this cut (two standard deviations under the N(0, 2) mean).
DISJOINT_CUT = -4.0


def load_calibration() -> dict:
    if not os.path.exists(CALIBRATION_FILE):
        return {}
    with open(CALIBRATION_FILE) as f:
        return json.load(f)


def draft_noise_scale(cid: int, override: float | None = None) -> float:
    """sigma (configs 2, 3) or c (config 5, noise sd = c * T_b) of the draft noise."""
    if override is not None:
        return float(override)
    if cid == 1:
        return CONFIG1_DRAFT_SD
    cal = load_calibration()
    key = str(cid)
    if key not in cal:
        raise RuntimeError(f"no calibrated draft noise for config {cid}; run oracle/calibrate_draft_noise.py")
    return float(cal[key]["scale"])


# --------------------------------------------------------------------------
# sampling-path inputs
# --------------------------------------------------------------------------
@dataclass
class SampleInputs:
    cfg: SampleConfig
    seed: int
    target: np.ndarray  # [B][gamma+1][V] uint16 (bf16 bits) or float32
    draft: np.ndarray  # [B][gamma][V]
    tokens: np.ndarray  # [B][gamma] int32
    uniforms: np.ndarray  # [B][gamma+1] float32
    temperature: np.ndarray  # [B] float32
    row_class: np.ndarray  # [B] int8: 0 normal, 1 disjoint, 2 identical
    extra: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.tokens.shape[0]

    @property
    def gamma(self):
        return self.tokens.shape[1]

    @property
    def V(self):
        return self.target.shape[-1]


def _to_dtype(a_f32: np.ndarray, dt: str) -> np.ndarray:
    return f32_to_bf16_bits(a_f32) if dt == "bf16" else np.ascontiguousarray(a_f32, dtype=np.float32)


def decode(a: np.ndarray, dt: str) -> np.ndarray:
    """Widen stored logits to float32 (exact)."""
    return bf16_bits_to_f32(a) if dt == "bf16" else np.asarray(a, dtype=np.float32)


def zipf_bias(seed: int, V: int, s: float = 1.1) -> np.ndarray:
    """Log-frequency bias -s*ln(rank) over one seeded permutation of [0, V)."""
    perm = gen(seed, 2, S_STRUCT).permutation(V)
    bias = np.empty(V, dtype=np.float64)
    bias[perm] = -s * np.log(np.arange(1, V + 1, dtype=np.float64))
    return bias


def target_rows(cfg: SampleConfig, seed: int, b: int, nrows: int, bias=None) -> np.ndarray:
    """float32 [nrows][V] target logits of sequence b, before dtype rounding."""
    g = gen(seed, cfg.cid, S_TARGET, b)
    z = g.standard_normal((nrows, cfg.V), dtype=np.float32) * np.float32(cfg.target_sd)
    if bias is not None:
        z = (z.astype(np.float64) + bias[None, :]).astype(np.float32)
    return z


def draft_rows(cfg: SampleConfig, seed: int, b: int, target_f32: np.ndarray, scale: float,
               row_class: int, T: float) -> np.ndarray:
    """float32 draft logits [gamma][V] of sequence b, built from the rounded target."""
    base = target_f32[: cfg.gamma]
    if row_class == 2:  # identical: exact copy of the (rounded) target
        return base.copy()
    if row_class == 1:  # support disjoint from the target's high-logit tokens
        out = base.copy()
        out[out >= np.float32(DISJOINT_CUT)] = -np.inf
        return out
    g = gen(seed, cfg.cid, S_DRAFT, b)
    sd = scale * T if cfg.cid == 5 else scale
    noise = g.standard_normal(base.shape, dtype=np.float32) * np.float32(sd)
    return base + noise


def row_classes(cfg: SampleConfig, seed: int) -> np.ndarray:
    cls = np.zeros(cfg.B, dtype=np.int8)
    if cfg.cid == 5:
        n_special = int(cfg.B * 0.1)
        perm = gen(seed, cfg.cid, S_STRUCT, 1).permutation(cfg.B)
        cls[perm[:n_special]] = 1
        cls[perm[n_special:2 * n_special]] = 2
    return cls


def temperatures(cfg: SampleConfig, seed: int, B: int) -> np.ndarray:
    t = cfg.temperature
    if isinstance(t, tuple):
        _, lo, hi = t
        return gen(seed, cfg.cid, S_STRUCT, 2).uniform(lo, hi, size=B).astype(np.float32)
    return np.full(B, t, dtype=np.float32)


def make_sample_inputs(cid: int, seed: int = 0, B: int | None = None, noise_scale: float | None = None,
                       trials: int | None = None, iid: bool = False) -> SampleInputs:
    """Build the inputs of sampling config ``cid`` (1, 2, 3 or 5).

    Config 1 (tiny): the logits are one seeded draw ([gamma+1][V] target,
    [gamma][V] draft) shared by every trial; each of ``trials`` sequences
    (default 10^4) gets its own draft tokens and uniforms. ``iid=True`` gives
    the variant whose rows are the same at every position (for the expected
    accepted length). The returned arrays then have leading dimension 1 and
    ``extra['shared_logits']`` is True: pass them with a sequence stride of 0.
    """
    cfg = CONFIGS[cid]
    assert isinstance(cfg, SampleConfig)
    if cid == 1:
        return _make_config1(seed, trials or 10_000, iid)
    if B is not None:
        cfg = SampleConfig(**{**cfg.__dict__, "B": B})
    scale = draft_noise_scale(cid, noise_scale)
    bias = zipf_bias(seed, cfg.V) if cid == 2 else None
    cls = row_classes(cfg, seed)
    temps = temperatures(cfg, seed, cfg.B)
    G, V = cfg.gamma, cfg.V
    tgt_store = np.empty((cfg.B, G + 1, V), dtype=np.uint16 if cfg.target_dtype == "bf16" else np.float32)
    dft_store = np.empty((cfg.B, G, V), dtype=np.uint16 if cfg.draft_dtype == "bf16" else np.float32)
    tokens = np.empty((cfg.B, G), dtype=np.int32)

    def one(b):
        t32 = target_rows(cfg, seed, b, G + 1, bias)
        tq = _to_dtype(t32, cfg.target_dtype)
        tgt_store[b] = tq
        t_round = decode(tq, cfg.target_dtype)
        d32 = draft_rows(cfg, seed, b, t_round, scale, int(cls[b]), float(temps[b]))
        dq = _to_dtype(d32, cfg.draft_dtype)
        dft_store[b] = dq
        d_round = decode(dq, cfg.draft_dtype).astype(np.float64)
        g = gen(seed, cfg.cid, S_DRAFTTOK, b)
        for i in range(G):
            tokens[b, i] = gumbel_max_draw(g, d_round[i], float(temps[b]))

    _pmap(one, range(cfg.B))
    u = uniforms_u24(gen(seed, cfg.cid, S_UNIFORM), (cfg.B, G + 1))
    return SampleInputs(cfg, seed, tgt_store, dft_store, tokens, u, temps, cls,
                        {"noise_scale": scale, "shared_logits": False})


def _make_config1(seed: int, trials: int, iid: bool) -> SampleInputs:
    cfg = CONFIGS[1]
    G, V = cfg.gamma, cfg.V
    g = gen(seed, 1, S_TARGET, 1 if iid else 0)
    nt = 1 if iid else G + 1
    t = g.standard_normal((nt, V), dtype=np.float32) * np.float32(cfg.target_sd)
    d = t[: (1 if iid else G)] + gen(seed, 1, S_DRAFT, 1 if iid else 0).standard_normal(
        (1 if iid else G, V), dtype=np.float32) * np.float32(CONFIG1_DRAFT_SD)
    if iid:
        t = np.repeat(t, G + 1, axis=0)
        d = np.repeat(d, G, axis=0)
    target = t[None].astype(np.float32)
    draft = d[None].astype(np.float32)
    dd = draft[0].astype(np.float64)
    gt = gen(seed, 1, S_DRAFTTOK, 1 if iid else 0)
    tokens = np.empty((trials, G), dtype=np.int32)
    # Each trial draws its drafts independently from the same q rows.
    for i in range(G):
        U = gt.random((trials, V))
        U[U == 0.0] = np.nextafter(0.0, 1.0)
        z = dd[i][None, :] / cfg.temperature - np.log(-np.log(U))
        tokens[:, i] = np.argmax(z, axis=1)
    u = uniforms_u24(gen(seed, 1, S_UNIFORM, 1 if iid else 0), (trials, G + 1))
    temps = np.full(trials, cfg.temperature, dtype=np.float32)
    return SampleInputs(cfg, seed, target, draft, tokens, u, temps, np.zeros(trials, np.int8),
                        {"noise_scale": CONFIG1_DRAFT_SD, "shared_logits": True, "iid": iid})


# --------------------------------------------------------------------------
# greedy-tree inputs
# --------------------------------------------------------------------------
@dataclass
class TreeInputs:
    cfg: TreeConfig
    seed: int
    logits: np.ndarray  # [B][N][V] uint16 (bf16 bits) or float32
    parents: np.ndarray  # [B][N] int32, parents[b][0] = -1, parents[b][j] < j
    tokens: np.ndarray  # [B][N] int32
    planted: np.ndarray  # [B][N] int8: 1 = an edge to a child was planted in row j
    dtype: str = "bf16"  # storage dtype of ``logits``


def tree_shape(g: np.random.Generator, N: int, block: int = 2, max_depth: int = 6,
               children=(2, 3, 4)) -> np.ndarray:
    """Parent array of a draft tree made of ``block``-token chains.

    The root and every node that ends a block (depth 0, block, 2*block, ...)
    gets a uniformly chosen number of child blocks from ``children``; a block is
    a chain of ``block`` nodes. Nodes are numbered level by level (BFS), the
    tree is cut to its first N nodes, and shapes with fewer than N nodes within
    ``max_depth`` are redrawn.
    """
    for _ in range(1000):
        nodes = [(-1, 0)]  # (parent, depth), appended level by level = BFS numbering
        frontier = [0]
        for _depth in range(max_depth):
            nxt = []
            for p in frontier:
                d = nodes[p][1]
                fan = int(g.choice(children)) if d % block == 0 else 1  # new blocks, or continue a chain
                for _c in range(fan):
                    nodes.append((p, d + 1))
                    nxt.append(len(nodes) - 1)
            frontier = nxt
        if len(nodes) >= N:
            parents = np.array([p for p, _ in nodes[:N]], dtype=np.int32)
            return parents
    raise RuntimeError("could not draw a tree with enough nodes")


def make_tree_inputs(cid: int = 4, seed: int = 0, B: int | None = None, N: int | None = None,
                     V: int | None = None, dtype: str | None = None) -> TreeInputs:
    """Build config-4 style inputs: draft trees plus target logits [B][N][V].

    Row j holds the target's next-token logits after node j. Target logits are
    N(0, 2) per element. For every node with children, with probability 0.75
    one child (uniformly chosen) has its token's logit in the node's row set
    to +16.0 (far above any N(0, 2) draw, so it becomes the row's top logit);
    otherwise +16.0 goes to a token that is no child's. Childless rows keep
    their natural top logit, where bf16 ties can occur. Sibling tokens are
    distinct.
    """
    cfg = CONFIGS[cid]
    assert isinstance(cfg, TreeConfig)
    B = B or cfg.B
    N = N or cfg.N
    V = V or cfg.V
    dtype = dtype or cfg.dtype
    logits = np.empty((B, N, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    parents = np.empty((B, N), dtype=np.int32)
    tokens = np.empty((B, N), dtype=np.int32)
    planted = np.zeros((B, N), dtype=np.int8)

    def one(b):
        gs = gen(seed, cid, S_STRUCT, b)
        par = tree_shape(gs, N, cfg.block, cfg.max_depth, cfg.children)
        kids = [[] for _ in range(N)]
        for j in range(1, N):
            kids[par[j]].append(j)
        tok = np.empty(N, dtype=np.int32)
        tok[0] = int(gs.integers(0, V))
        for p in range(N):
            if kids[p]:
                tok[kids[p]] = gs.choice(V, size=len(kids[p]), replace=False).astype(np.int32)
        z = gen(seed, cid, S_TARGET, b).standard_normal((N, V), dtype=np.float32) * np.float32(cfg.target_sd)
        for p in range(N):
            if not kids[p]:
                continue
            if gs.random() < cfg.plant_prob:
                c = kids[p][int(gs.integers(0, len(kids[p])))]
                z[p, tok[c]] = cfg.plant_value
                planted[b, p] = 1
            else:
                child_toks = set(int(tok[c]) for c in kids[p])
                while True:
                    t = int(gs.integers(0, V))
                    if t not in child_toks or len(child_toks) >= V:
                        break
                z[p, t] = cfg.plant_value
        logits[b] = _to_dtype(z, dtype)
        parents[b] = par
        tokens[b] = tok

    _pmap(one, range(B))
    return TreeInputs(cfg, seed, logits, parents, tokens, planted, dtype)


def make_custom_sample(B: int, gamma: int, V: int, target_dtype: str = "bf16", draft_dtype: str = "bf16",
                       T=1.0, noise_sd: float = 0.8, target_sd: float = 2.0, seed: int = 0,
                       cid: int = 100) -> SampleInputs:
    """Generic sampling inputs: target N(0, target_sd), draft = rounded target +
    N(0, noise_sd), drafts x ~ q (Gumbel-max), exact u24 uniforms. ``T`` is a
    float or an array of B temperatures."""
    temps = np.broadcast_to(np.asarray(T, dtype=np.float32), (B,)).copy()
    cfg = SampleConfig(cid, "custom", B, gamma, V, target_dtype, draft_dtype, target_sd, float(temps[0]))
    tgt = np.empty((B, gamma + 1, V), dtype=np.uint16 if target_dtype == "bf16" else np.float32)
    dft = np.empty((B, gamma, V), dtype=np.uint16 if draft_dtype == "bf16" else np.float32)
    tokens = np.empty((B, gamma), dtype=np.int32)

    def one(b):
        t32 = target_rows(cfg, seed, b, gamma + 1)
        tq = _to_dtype(t32, target_dtype)
        tgt[b] = tq
        tr = decode(tq, target_dtype)[:gamma]
        z = gen(seed, cid, S_DRAFT, b).standard_normal(tr.shape, dtype=np.float32)
        dq = _to_dtype(tr + z * np.float32(noise_sd), draft_dtype)
        dft[b] = dq
        dr = decode(dq, draft_dtype).astype(np.float64)
        g = gen(seed, cid, S_DRAFTTOK, b)
        for i in range(gamma):
            tokens[b, i] = gumbel_max_draw(g, dr[i], float(temps[b]))

    _pmap(one, range(B))
    u = uniforms_u24(gen(seed, cid, S_UNIFORM), (B, gamma + 1))
    return SampleInputs(cfg, seed, tgt, dft, tokens, u, temps, np.zeros(B, np.int8), {"shared_logits": False})


# --------------------------------------------------------------------------
# draft-side sampler inputs
# --------------------------------------------------------------------------
@dataclass
class DraftRows:
    name: str
    seed: int
    dtype: str
    logits: np.ndarray       # [B][V]: bf16 bits (uint16) or float32
    uniforms: np.ndarray     # [B] float32, exact k * 2^-24
    temperature: np.ndarray  # [B] float32

    @property
    def B(self):
        return self.logits.shape[0]

    @property
    def V(self):
        return self.logits.shape[1]


def make_draft_rows(B: int, V: int, dtype: str = "f32", T=1.0, seed: int = 0, sd: float = 2.0,
                    cid: int = 200, name: str = "custom draft rows") -> DraftRows:
    """One draft logit row per sequence, N(0, sd), rounded to dtype; one exact
    u24 uniform per row; T a float or B temperatures."""
    temps = np.broadcast_to(np.asarray(T, dtype=np.float32), (B,)).copy()
    out = np.empty((B, V), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(b):
        z = gen(seed, cid, S_TARGET, b).standard_normal(V, dtype=np.float32) * np.float32(sd)
        out[b] = _to_dtype(z, dtype)

    _pmap(one, range(B))
    u = uniforms_u24(gen(seed, cid, S_UNIFORM), (B,))
    return DraftRows(name, seed, dtype, out, u, temps)


def make_draft_workload(cid: int, seed: int = 0) -> DraftRows:
    """The draft sampler's share of sampling configuration cid: B rows of V
    draft logits in the configuration's draft dtype and temperatures."""
    cfg = CONFIGS[cid]
    return make_draft_rows(cfg.B, cfg.V, cfg.draft_dtype, temperatures(cfg, seed, cfg.B), seed, cfg.target_sd,
                           cid=200 + cid, name=f"draft rows of config {cid}")


# --------------------------------------------------------------------------
# synthetic Markov-chain models (end-to-end loop)
# --------------------------------------------------------------------------
@dataclass
class MarkovTables:
    """Next-token logits of a first-order Markov 'target model' and a perturbed
    'draft model': row s holds the logits after token s. Stored in dtype."""
    V: int
    dtype: str
    target: np.ndarray  # [V][V]
    draft: np.ndarray   # [V][V]
    seed: int


def make_markov_tables(V: int, dtype: str = "f32", seed: int = 0, target_sd: float = 2.0,
                       noise_sd: float = 0.8, cid: int = 300) -> MarkovTables:
    st = np.uint16 if dtype == "bf16" else np.float32
    tq = np.empty((V, V), dtype=st)
    dq = np.empty((V, V), dtype=st)

    def rows(r0):  # one generator per block of 64 rows, so blocks run in parallel
        r1 = min(V, r0 + 64)
        t32 = gen(seed, cid, S_TARGET, r0).standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(target_sd)
        tq[r0:r1] = _to_dtype(t32, dtype)
        z = gen(seed, cid, S_DRAFT, r0).standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(noise_sd)
        dq[r0:r1] = _to_dtype(decode(tq[r0:r1], dtype) + z, dtype)

    _pmap(rows, range(0, V, 64))
    return MarkovTables(V, dtype, tq, dq, seed)


def tree_blocks(parents: np.ndarray, block: int = 2) -> np.ndarray:
    """Block ids of a draft tree built by tree_shape: the nodes a drafter
    proposes together in one block of ``block`` tokens share an id (the index
    of the block's first node); a node at depth d >= 1 starts a block when
    (d - 1) is a multiple of ``block``, else it continues its parent's. The
    root (the already accepted token) has id -1."""
    N = len(parents)
    depth = np.zeros(N, dtype=np.int64)
    blk = np.full(N, -1, dtype=np.int32)
    for j in range(1, N):
        p = int(parents[j])
        depth[j] = depth[p] + 1
        blk[j] = j if (depth[j] - 1) % block == 0 else blk[p]
    return blk
