#!/usr/bin/env python3
"""Benchmark of the verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

A step is one pass of the whole hot path over one batch: spec_verify_sample
(row statistics + accept tests + first rejection, then the residual/bonus draw)
for the sampling workloads, spec_verify_greedy_tree for the tree workload.
Inputs are seeded synthetic logits already resident in HBM. Prints ONE JSON
line on stdout; progress goes to stderr. Without --steps / --warmup the
untimed warm-up lasts about 0.3 s of the same work and the timed pass about
0.2 s (at least 20 steps each); the line reports the counts used.

Workloads d3, d5 time the draft-side sampler (spec_draft_sample) on the draft
rows of configurations 3 and 5 (256 x 128256 bf16 at T 0.7; 512 x 256000
fp32 at per-row T); they print the same kind of line with their own metric.

Workload m runs the end-to-end loop on a synthetic Markov-chain model pair
(512 chains, V = 16384 bf16 transition-logit tables, gamma = 5, T = 1): per
iteration gamma draft-sampler calls, the target-row gathers and one verify;
value = emitted tokens per second.

Workloads t4 and t1024 time the draft-tree mask builder (spec_tree_mask: tree
mask, relaxed block mask and depths): the configuration-4 trees (32 x 60
nodes, 2-token blocks) and 32 random trees of 1024 nodes.

Workloads (the five input configurations): c1 tiny sampling (B=10^4 trials,
gamma=4, V=32, fp32), c2 7B-class vocab (B=64, gamma=4, V=32000, bf16), c3
large vocab (B=256, gamma=8, V=128256, bf16, T=0.7), c4 greedy tree (B=32,
N=60, V=32000, bf16), c5 stress (B=512, gamma=5, V=256000, bf16 target, fp32
draft, per-row T in [0.3, 1.5]). The default is c5, the largest single-GPU one.
b3 and b5 run configurations 3 and 5 at a batch of one sequence; s3 and s5 at
32 and 64 sequences, one GPU's share of the batch split by sequence over eight.

--calibrate-copy runs a plain 1 GiB device-to-device copy instead (used to
scale the FETCH_SIZE / WRITE_SIZE counters of rocprofv3 runs). For the
sampling workloads the line's detail also times spec_verify_sample_early_exit
on the same inputs (rows after a first rejection are not read; algorithmic
bytes counted for the rows it must read); --early-exit makes that entry point
the timed step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBPS = float(os.environ.get("SV_PEAK_HBM_GBPS", "8000"))
WORKLOADS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "d3": 3, "d5": 5, "m": 0, "t4": 4, "t1024": 4,
             "b3": 3, "b5": 5, "s3": 3, "s5": 5}
# Batch sizes other than the configuration's: b3, b5 are configurations 3 and 5
# at a batch of one sequence (latency); s3, s5 at one eighth of their batch
# (32 and 64 sequences), the share of one GPU when the batch is split by
# sequence over eight.
BATCH = {"b3": 1, "b5": 1, "s3": 32, "s5": 64}
MARKOV = dict(B=512, V=16384, gamma=5, T=1.0, dtype="bf16", noise_sd=0.8)
CSRC = os.path.join(ROOT, "lossless_draft_verification_05_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Untimed and timed work when --warmup / --steps are not given: the GPU
# settles over tens of milliseconds of sustained work (after 3 untimed steps
# c3's finish kernel still ran 28% slower than after 300), so the warm-up runs
# for about WARM_S seconds of the same work and the timed pass for about
# TIMED_S seconds, each at least MIN_STEPS steps.
WARM_S, TIMED_S, MIN_STEPS = 0.3, 0.2, 20


def warm_up(call, args):
    """Runs the untimed steps call(0), call(1), ...: args.warmup of them. A
    missing args.warmup or args.steps is set first from the time of up to
    three untimed calls (counted in the warm-up)."""
    import torch

    done = 0
    if args.warmup is None or args.steps is None:
        n_probe = 3 if args.warmup is None else min(3, args.warmup)
        if n_probe > 0:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(n_probe):
                call(k)
            torch.cuda.synchronize()
            est = max((time.perf_counter() - t0) / n_probe, 1e-6)
        else:
            est = TIMED_S / MIN_STEPS
        done = n_probe
        if args.warmup is None:
            args.warmup = max(MIN_STEPS, int(np.ceil(WARM_S / est)))
        if args.steps is None:
            args.steps = max(MIN_STEPS, int(np.ceil(TIMED_S / est)))
    for k in range(done, args.warmup):
        call(k)
    torch.cuda.synchronize()


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands, on a bounded sample
# ----------------------------------------------------------------------------
_CPU_DATA = None


def _oracle_seq(b):
    from oracle import spec_verify_oracle as O

    inp, tdt, ddt = _CPU_DATA
    lb = 0 if inp.target.shape[0] != inp.tokens.shape[0] else b
    r = O.verify_sample_sequence(O.widen(inp.target[lb], tdt), O.widen(inp.draft[lb], ddt), inp.tokens[b],
                                 inp.uniforms[b].astype(np.float64), float(inp.temperature[b]))
    return r.n


def _oracle_tree(b):
    from oracle import spec_verify_oracle as O

    ti = _CPU_DATA
    return O.verify_tree_sequence(O.widen(ti.logits[b], ti.dtype), ti.parents[b], ti.tokens[b]).accept_len


def _oracle_draft(b):
    from oracle import spec_verify_oracle as O

    d = _CPU_DATA
    return O.draft_sample_row(O.widen(d.logits[b], d.dtype), float(d.temperature[b]), float(d.uniforms[b])).y


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


# The oracle's worker pool: at most 16 processes, the CPU share of one GPU on
# the benchmark host (os.cpu_count() there reports the whole machine).
MAX_ORACLE_WORKERS = 16


def time_oracle(fn, n_items: int, units, unit: str, what: str, budget_s: float = 10.0, cap: int = 2_000_000):
    """Time the oracle function fn(i) (item i mod n_items of the same inputs)
    once in this process on about budget_s / 4 seconds of work, and once in a
    pool of worker processes (forked before the GPU is touched) on about
    budget_s seconds. units: units of the metric per item, or None when fn
    returns its item's units. The pool's rate is the baseline's value."""
    import multiprocessing as mp

    fn(0)  # warm (imports, first touch)
    t0 = time.perf_counter()
    fn(0)
    t_one = max(time.perf_counter() - t0, 1e-5)

    def count(results, items):
        return sum(results) if units is None else units * items

    s1 = int(min(cap, max(1, 0.25 * budget_s / t_one)))
    t0 = time.perf_counter()
    r1 = [fn(i % n_items) for i in range(s1)]
    dt1 = time.perf_counter() - t0
    workers = max(1, min(MAX_ORACLE_WORKERS, os.cpu_count() or 1))
    S = int(min(cap, max(workers, budget_s * workers / t_one)))
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        res = pool.map(fn, [i % n_items for i in range(S)], chunksize=max(1, S // (4 * workers)))
        dt = time.perf_counter() - t0
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = None
    return {"value": count(res, S) / dt, "unit": unit, "cores": workers, "kind": "oracle",
            "sample": f"{S} {what} (index mod {n_items}) of the same inputs, {workers} worker processes, {dt:.1f} s",
            "single_process": {"value": count(r1, s1) / dt1, "unit": unit,
                               "sample": f"{s1} {what}, one process, {dt1:.1f} s"},
            "cpu_count": os.cpu_count(), "cpus_available": avail, "cpu_model": _cpu_model(),
            "pool_cap": f"{MAX_ORACLE_WORKERS} worker processes at most: the CPU share of one GPU on the "
                        f"benchmark host"}


def cpu_baseline_draft(d, budget_s: float = 10.0):
    """The oracle's draft sampler over a bounded sample of rows (cycled)."""
    global _CPU_DATA
    _CPU_DATA = d
    out = time_oracle(_oracle_draft, d.B, 1, "draft tokens/s", "rows (numpy fp64)", budget_s)
    _CPU_DATA = None
    return out


def bench_draft(args, cid):
    """Time spec_draft_sample (the one-pass kernel where it applies, HIP events
    on the stream it runs on) on the draft rows of configuration cid, and the
    staged two-kernel path beside it."""
    log(f"[bench] building draft rows of config {cid} (seed {args.seed})")
    d = synth.make_draft_workload(cid, seed=args.seed)
    cpu = None if args.no_cpu_baseline else cpu_baseline_draft(d)
    if cpu:
        log(f"[bench] cpu baseline: {cpu}")
    import torch

    from lossless_draft_verification_05_amd import binding

    binding.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    a = np.ascontiguousarray(d.logits)
    L0 = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev) if d.dtype == "bf16" else \
        torch.from_numpy(a).to(dev)
    per_copy = L0.numel() * L0.element_size()
    R = int(min(64, max(1, -(-(512 << 20) // per_copy)))) if per_copy < (512 << 20) else 1
    copies = [L0] + [L0.clone() for _ in range(R - 1)]
    u = torch.from_numpy(d.uniforms).to(dev)
    T = torch.from_numpy(d.temperature).to(dev)
    y = torch.empty(d.B, dtype=torch.int32, device=dev)
    ws = binding.Workspace()

    def timed(calls_of):
        """mean ms per step (wall clock over a pass with nothing else on the
        stream) and per-call HIP-event means (ms, from a second pass)"""
        def step(k):
            for f in calls_of(k % R):
                f()
        warm_up(step, args)
        t0 = time.perf_counter()
        for k in range(args.steps):
            for f in calls_of(k % R):
                f()
        torch.cuda.synchronize()
        ms_ = (time.perf_counter() - t0) * 1e3 / args.steps
        n = len(calls_of(0))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.steps)]
        for k in range(args.steps):
            e = evs[k]
            e[0].record()
            for i, f in enumerate(calls_of(k % R)):
                f()
                e[i + 1].record()
        torch.cuda.synchronize()
        return ms_, [float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
                     for i in range(n)]

    one_pass = d.B >= 128 or d.V * (2 if d.dtype == "bf16" else 4) <= (64 << 10)
    # calls prepared once (arguments checked and marshalled), so the timed loops
    # measure the GPU, not the Python binding
    one = [[binding.spec_draft_sample(copies[c], u, T, out_tokens=y, workspace=ws, prepare=True)] for c in range(R)]
    two = [[binding.spec_draft_sample(copies[c], u, T, out_tokens=y, workspace=ws, stage=s, prepare=True)
            for s in (1, 2)] for c in range(R)]
    ms, st = timed(lambda c: one[c])
    log(f"[bench] {ms:.4f} ms/step; kernel event mean (ms): {st}")
    ms2, st2 = timed(lambda c: two[c])
    log(f"[bench] staged (two kernels): {ms2:.4f} ms/step; kernel event means (ms): {st2}")
    row_bytes = d.V * (2 if d.dtype == "bf16" else 4)
    step_bytes = min(d.V, 2048) * (2 if d.dtype == "bf16" else 4)
    s1 = d.B * row_bytes + d.B * 8          # every logit once + temperatures, uniforms
    s_draw = d.B * step_bytes + d.B * 4     # the rescanned step + the tokens
    sha = kernel_source_sha()
    kname = "sv_draft1_kernel" if one_pass else "sv_stats_kernel + sv_finish_kernel"
    alg = s1 + s_draw if one_pass else 2 * s1 + s_draw
    achieved = alg / (st[0] * 1e-3) / 1e9
    yy = y.cpu().numpy()
    line = {
        "metric": "sampled draft tokens/sec + achieved HBM GB/s (% peak), spec_draft_sample at 1 GPU",
        "value": d.B / (ms * 1e-3), "unit": "draft tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic: seeded logits standing in for draft model outputs",
        "config": {"workload": f"{args.workload}: draft rows of configuration {cid}", "B": d.B, "V": d.V,
                   "dtype": d.dtype, "seed": args.seed},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_from_profiles(args.workload, sha)},
        "cpu_baseline": cpu,
        "detail": {"kernels": {kname: {"mean_us": round(st[0] * 1e3, 3), "alg_bytes": alg,
                                       "gbps": round(achieved, 1)}},
                   "two_kernel_path": {"ms_per_step": ms2,
                                       "sv_stats_kernel_us": round(st2[0] * 1e3, 3),
                                       "sv_finish_kernel_us": round(st2[1] * 1e3, 3),
                                       "alg_bytes": 2 * s1 + s_draw},
                   "input_copies": R, "kernel_source_sha": sha, "invalid": int((yy < 0).sum())},
    }
    print(json.dumps(line), flush=True)


def _oracle_markov(job):
    from oracle import spec_verify_oracle as O

    tabs, T, K, G = _CPU_DATA
    b = job
    g = np.random.default_rng(1000 + b)
    res = O.markov_loop(tabs[0], tabs[1], T, b % tabs[0].shape[0], g.random((K, G)), g.random((K, G + 1)))
    return sum(n + 1 for n, _ in res)


def bench_markov(args):
    """End-to-end loop on a Markov-chain model pair: emitted tokens per second
    (HIP events around the timed iterations on the current stream)."""
    from oracle import spec_verify_oracle as O  # noqa: F401  (CPU baseline only)

    c = MARKOV
    B, V, G, T = c["B"], c["V"], c["gamma"], c["T"]
    log(f"[bench] building Markov tables V={V} ({c['dtype']}, seed {args.seed})")
    tabs = synth.make_markov_tables(V, c["dtype"], seed=args.seed, noise_sd=c["noise_sd"])
    cpu = None
    if not args.no_cpu_baseline:
        global _CPU_DATA
        Lt = synth.decode(tabs.target, c["dtype"]).astype(np.float64)
        Ld = synth.decode(tabs.draft, c["dtype"]).astype(np.float64)
        K = 4
        _CPU_DATA = ((Lt, Ld), T, K, G)
        cpu = time_oracle(_oracle_markov, 4 * B, None, "emitted tokens/s",
                          f"chains x {K} iterations of the oracle loop (draft_sample_row + verify_sample_sequence, "
                          f"numpy fp64)", cap=4 * B)
        _CPU_DATA = None
        log(f"[bench] cpu baseline: {cpu}")
    import torch

    from lossless_draft_verification_05_amd import binding
    from lossless_draft_verification_05_amd.markov import MarkovLoop

    binding.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a):
        a = np.ascontiguousarray(a)
        if c["dtype"] == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    loop = MarkovLoop(up(tabs.target), up(tabs.draft), G, torch.full((B,), T, dtype=torch.float32, device=dev))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    if args.warmup is None:
        args.warmup = 50
    if args.steps is None:
        args.steps = 20
    n_it = args.warmup + args.steps
    ud = torch.rand((n_it, B, G), generator=gen, device=dev)
    uv = torch.rand((n_it, B, G + 1), generator=gen, device=dev)
    state = torch.arange(B, device=dev, dtype=torch.int64) % V
    emitted = torch.zeros((), dtype=torch.int64, device=dev)
    loop.capture(state, ud[0], uv[0])  # one iteration as a HIP graph (replayed below)
    loop.g_state.copy_(state)
    for k in range(args.warmup):  # the same work as a timed iteration (loads every kernel it uses)
        n, _ = loop.replay(ud[k], uv[k])
        emitted += (n.long() + 1).sum()
    torch.cuda.synchronize()
    emitted.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for k in range(args.warmup, n_it):
        n, _ = loop.replay(ud[k], uv[k])
        emitted += (n.long() + 1).sum()
    e1.record()
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    tok = int(emitted.item())
    esz_ = 2 if c["dtype"] == "bf16" else 4
    # hot-path bytes per iteration: gamma draft-sampler calls (row read twice) + the verify's one pass over
    # 2 gamma + 1 rows + its draw row(s) (counted as a row pair)
    it_bytes = B * V * esz_ * (2 * G + (2 * G + 1) + 2)
    achieved = it_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "emitted tokens/sec, end-to-end speculative decoding on a Markov-chain model pair "
                  "(spec_draft_sample + spec_verify_sample) at 1 GPU",
        "value": tok / (args.steps * ms * 1e-3), "unit": "emitted tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic: seeded Markov transition-logit tables",
        "config": {"workload": "m: Markov-chain loop", "B": B, "V": V, "gamma": G, "temperature": T,
                   "table_dtype": c["dtype"], "seed": args.seed},
        "roofline": {"bound": "hbm", "kernel": "whole iteration (gamma draft-sampler calls, row gathers, verify)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "detail": {"tokens_per_call": tok / (args.steps * B), "ms_per_step_wall": ms_wall,
                   "launch": "one captured HIP graph per iteration",
                   "hot_path_bytes_per_iteration": it_bytes, "kernel_source_sha": kernel_source_sha()},
    }
    print(json.dumps(line), flush=True)


def _oracle_masks(b):
    from oracle import spec_verify_oracle as O

    P, Bl = _CPU_DATA
    O.tree_masks(P[b], Bl[b])
    return 1


def bench_masks(args):
    """spec_tree_mask on the configuration-4 trees (t4) or 32 random
    1024-node trees (t1024); HIP events around each call."""
    if args.workload == "t4":
        ti = synth.make_tree_inputs(4, seed=args.seed)
        P = ti.parents
        desc = "t4: masks of the configuration-4 draft trees"
    else:
        g = synth.gen(args.seed, 4, 2, 1024)
        P = np.stack([[-1] + [int(g.integers(max(0, j - 16), j)) for j in range(1, 1024)] for _ in range(32)])
        P = P.astype(np.int32)
        desc = "t1024: masks of 32 random 1024-node trees"
    Bl = np.stack([synth.tree_blocks(p) for p in P]).astype(np.int32)
    B, N = P.shape
    cpu = None
    if not args.no_cpu_baseline:
        global _CPU_DATA
        _CPU_DATA = (P, Bl)
        cpu = time_oracle(_oracle_masks, B, 1, "trees/s", "trees (python loops)", cap=200_000)
        _CPU_DATA = None
        log(f"[bench] cpu baseline: {cpu}")
    import torch

    from lossless_draft_verification_05_amd import binding

    binding.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    Pt, Blt = torch.from_numpy(P).to(dev), torch.from_numpy(Bl).to(dev)
    R = int(min(64, max(1, -(-(512 << 20) // (2 * B * N * N)))))
    outs = [(torch.empty((B, N, N), dtype=torch.uint8, device=dev), torch.empty((B, N, N), dtype=torch.uint8,
             device=dev), torch.empty((B, N), dtype=torch.int32, device=dev)) for _ in range(R)]

    prep = [binding.spec_tree_mask(Pt, Blt, want_relaxed=True, out_mask=m, out_relaxed=r, out_depth=d, prepare=True)
            for m, r, d in outs]

    def call(k):
        prep[k % R]()
    warm_up(call, args)
    # timed pass with nothing else on the stream, then a pass with HIP events
    t0 = time.perf_counter()
    for k in range(args.steps):
        call(k)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for k in range(args.steps):
        evs[k][0].record()
        call(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    kern = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    kname = "sv_mask64_kernel" if N <= 64 else "sv_mask_kernel"  # trees of at most 64 nodes: one wave per tree
    nbytes = 2 * B * N * N + B * N * 4 * 3  # both masks written, parents and blocks read, depths written
    achieved = nbytes / (kern * 1e-3) / 1e9
    line = {
        "metric": "draft-tree masks/sec + achieved HBM GB/s (% peak), spec_tree_mask at 1 GPU",
        "value": B / (ms * 1e-3), "unit": "trees/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic: seeded draft-tree parent arrays",
        "config": {"workload": desc, "B": B, "N": N, "block": 2, "seed": args.seed},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_from_profiles(args.workload, kernel_source_sha())},
        "cpu_baseline": cpu,
        "detail": {"kernels": {kname: {"mean_us": round(kern * 1e3, 3), "alg_bytes": nbytes}},
                   "output_copies": R, "kernel_source_sha": kernel_source_sha()},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(inp, tree: bool, budget_s: float = 10.0):
    """Time the oracle over sequences (trees) of the same inputs, cycled when
    the batch takes less than the budget (see time_oracle)."""
    global _CPU_DATA
    _CPU_DATA = inp if tree else (inp, inp.cfg.target_dtype, inp.cfg.draft_dtype)
    if tree:
        out = time_oracle(_oracle_tree, inp.parents.shape[0], inp.parents.shape[1] - 1, "nodes/s",
                          "trees (numpy fp64)", budget_s)
    else:
        out = time_oracle(_oracle_seq, inp.tokens.shape[0], inp.tokens.shape[1], "positions/s",
                          "sequences (numpy fp64)", budget_s)
    _CPU_DATA = None
    return out


# ----------------------------------------------------------------------------
# algorithmic bytes
# ----------------------------------------------------------------------------
def esz(dt):
    return 2 if dt == "bf16" else 4


def sample_bytes(cfg, B, G, V, n_acc=None):
    """(stats-kernel bytes, finish-kernel bytes) the method must move per call.

    The stats kernel reads every target and draft logit once (plus tokens,
    uniforms and temperatures, counted with it). The finish kernel reads the
    one row the draw needs again -- target and draft row n after a rejection,
    target row gamma after full acceptance -- and writes the outputs."""
    bt, bd = esz(cfg.target_dtype), esz(cfg.draft_dtype)
    s1 = B * ((G + 1) * V * bt + G * V * bd) + B * (G * 4 + (G + 1) * 4 + 4)
    if n_acc is None:
        s2 = None
    else:
        rej = int((n_acc < G).sum())
        s2 = rej * V * (bt + bd) + (B - rej) * V * bt + B * (G + 2) * 4
    return s1, s2


def early_exit_bytes(cfg, B, G, V, n_acc):
    """Bytes the early-exit path must move: target rows 0..n and draft rows
    0..min(n, gamma-1) of every sequence (all rows for an invalid one), the
    draw row(s) again, per-position inputs and outputs."""
    bt, bd = esz(cfg.target_dtype), esz(cfg.draft_dtype)
    n = np.where(n_acc < 0, G, n_acc).astype(np.int64)
    stats = int(((n + 1) * V * bt + (np.minimum(n, G - 1) + 1) * V * bd).sum())
    _, s2 = sample_bytes(cfg, B, G, V, n_acc)
    return stats + s2 + B * (G * 4 + (G + 1) * 4 + 4)


# ----------------------------------------------------------------------------
def traffic_from_profiles(workload: str, sha: str):
    # profiles/<dominant kernel>_<workload>_traffic.json
    import glob
    found = glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_traffic.json"))
    if len(found) != 1:
        return None
    path = found[0]
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None
    return t.get("hbm_bytes_per_launch")


def run_copy_calibration():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    # default: about WARM_S seconds of untimed steps and TIMED_S seconds of
    # timed ones (see warm_up); the counts are reported
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--early-exit", action="store_true",
                    help="time spec_verify_sample_early_exit (rows after a first rejection are not read)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the verify step shards by sequence "
                                   "with no exchange, and no multi-GPU figure is produced",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.calibrate_copy:
        run_copy_calibration()
        return

    cid = WORKLOADS[args.workload]
    if args.workload == "m":
        bench_markov(args)
        return
    if args.workload.startswith("t"):
        bench_masks(args)
        return
    if args.workload.startswith("d"):
        bench_draft(args, cid)
        return
    tree = cid == 4
    log(f"[bench] building inputs for {args.workload} (seed {args.seed})")
    t0 = time.perf_counter()
    inp = synth.make_tree_inputs(4, seed=args.seed) if tree else \
        synth.make_sample_inputs(cid, seed=args.seed, B=BATCH.get(args.workload))
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a bounded sample")
        cpu = cpu_baseline(inp, tree)
        log(f"[bench] cpu baseline: {cpu}")

    import torch

    from lossless_draft_verification_05_amd import binding

    binding.load()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(dev)

    # copies so that workloads smaller than the 256 MB Infinity Cache are not
    # served from it across steps
    if tree:
        per_copy = inp.logits.nbytes
    else:
        per_copy = inp.target.nbytes + inp.draft.nbytes
    R = int(min(64, max(1, -(-(512 << 20) // per_copy)))) if per_copy < (512 << 20) else 1
    log(f"[bench] uploading {R} input cop{'y' if R == 1 else 'ies'} of {per_copy / 1e6:.1f} MB")
    sha = kernel_source_sha()
    if tree:
        L = up(inp.logits, inp.dtype)
        copies = [L] + [L.clone() for _ in range(R - 1)]
        par = torch.from_numpy(inp.parents).to(dev)
        tok = torch.from_numpy(inp.tokens).to(dev)
        B, N, V = inp.logits.shape
        ws = binding.Workspace()
        outs = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev))

        # calls prepared once (arguments checked and marshalled), so the timed
        # loop measures the GPU, not the Python binding
        prep = {(s, c): binding.spec_verify_greedy_tree_stage(s, copies[c], par, tok, out_accept_len=outs[0],
                                                               out_path=outs[1], out_bonus=outs[2],
                                                               out_argmax=outs[3], workspace=ws, prepare=True)
                for s in (1, 2) for c in range(R)}

        whole = [binding.spec_verify_greedy_tree(copies[c], par, tok, out_accept_len=outs[0], out_path=outs[1],
                                                 out_bonus=outs[2], out_argmax=outs[3], workspace=ws, prepare=True)
                 for c in range(R)]

        def stages(c):
            return [prep[(1, c)], prep[(2, c)]]
        units = B * (N - 1)
        unit = "nodes/s"
        s1_bytes = B * N * V * esz(inp.dtype) + 2 * B * N * 4
        cfg_desc = {"workload": f"{args.workload}: greedy decoding-tree verification", "B": B, "N": N, "V": V,
                    "logits_dtype": inp.dtype, "seed": args.seed}
        # trees of at most 64 nodes resolve in one wave (no LDS, no barrier)
        kernel_names = ["sv_argmax_kernel", "sv_tree64_kernel" if N <= 64 else "sv_tree_kernel"]
    else:
        cfg = inp.cfg
        t0_ = up(inp.target, cfg.target_dtype)
        d0_ = up(inp.draft, cfg.draft_dtype)
        B = inp.tokens.shape[0]
        tcopies = [t0_] + [t0_.clone() for _ in range(R - 1)]
        dcopies = [d0_] + [d0_.clone() for _ in range(R - 1)]
        if t0_.shape[0] != B:  # shared logits (c1): stride-0 batch dimension
            tcopies = [t.expand(B, *t.shape[1:]) for t in tcopies]
            dcopies = [d.expand(B, *d.shape[1:]) for d in dcopies]
        tokens = torch.from_numpy(inp.tokens).to(dev)
        uni = torch.from_numpy(inp.uniforms).to(dev)
        temps = torch.from_numpy(inp.temperature).to(dev)
        G, V = inp.tokens.shape[1], inp.target.shape[-1]
        ws = binding.Workspace()
        out_n = torch.empty(B, dtype=torch.int32, device=dev)
        out_t = torch.empty((B, G + 1), dtype=torch.int32, device=dev)

        # calls prepared once (arguments checked and marshalled), so the timed
        # loop measures the GPU, not the Python binding
        if args.early_exit:
            prep = {c: [binding.spec_verify_sample_early_exit(tcopies[c], dcopies[c], tokens, uni, temps,
                                                              out_num_accepted=out_n, out_tokens=out_t,
                                                              workspace=ws, prepare=True)] for c in range(R)}
        else:
            prep = {c: [binding.spec_verify_sample_stage(k, tcopies[c], dcopies[c], tokens, uni, temps,
                                                         out_num_accepted=out_n, out_tokens=out_t, workspace=ws,
                                                         prepare=True) for k in (1, 2)] for c in range(R)}
        whole = [prep[c][0] if args.early_exit else
                 binding.spec_verify_sample(tcopies[c], dcopies[c], tokens, uni, temps, out_num_accepted=out_n,
                                            out_tokens=out_t, workspace=ws, prepare=True) for c in range(R)]

        def stages(c):
            return prep[c]
        units = B * G
        unit = "positions/s"
        s1_bytes, _ = sample_bytes(cfg, B, G, V)
        tdesc = cfg.temperature if not isinstance(cfg.temperature, tuple) else f"U[{cfg.temperature[1]}, {cfg.temperature[2]}] per row"
        nb = BATCH.get(args.workload)
        cfg_desc = {"workload": f"{args.workload}: {cfg.name}" + (f" at a batch of {nb}" if nb else ""),
                    "B": B, "gamma": G, "V": V,
                    "target_dtype": cfg.target_dtype, "draft_dtype": cfg.draft_dtype, "temperature": tdesc,
                    "seed": args.seed}
        kernel_names = ["sv_stats_kernel", "sv_finish_kernel"]
        small = V <= 2048 and not args.early_exit  # the full call is one kernel, a wave per sequence
        if small:
            # two sequences per wave when a row fits half a wave and so do the 2 gamma + 1 row slots
            kernel_names = ["sv_small2_kernel" if V <= 32 and 2 * G + 1 <= 32 else "sv_small_kernel"]
            prep = {c: [whole[c]] for c in range(R)}
        if args.early_exit:
            kernel_names = ["spec_verify_sample_early_exit"]
            cfg_desc["entry_point"] = "spec_verify_sample_early_exit"

    torch.cuda.synchronize()
    warm_up(lambda k: whole[k % R](), args)
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    # The timed pass: whole calls, nothing else on the stream (an event
    # recorded between two kernels costs 10-20 us of GPU time per step here).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        whole[k % R]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # A second pass of as many steps, kernel by kernel with HIP events between
    # them on the stream the kernels run on: the per-kernel durations.
    ns = len(stages(0))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        fs = stages(k % R)
        e = evs[k]
        e[0].record()
        for i, f in enumerate(fs):
            f()
            e[i + 1].record()
    torch.cuda.synchronize()

    # the early-exit entry point on the same inputs, timed the same way (reported in detail)
    ee = None
    if not tree and not args.early_exit:
        ee_n = torch.empty_like(out_n)
        ee_t = torch.empty_like(out_t)
        ee_prep = [binding.spec_verify_sample_early_exit(tcopies[c], dcopies[c], tokens, uni, temps,
                                                         out_num_accepted=ee_n, out_tokens=ee_t, workspace=ws,
                                                         prepare=True) for c in range(R)]

        def ee_call(c):
            ee_prep[c]()
        for k in range(args.warmup):
            ee_call(k % R)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for k in range(args.steps):
            ee_call(k % R)
        torch.cuda.synchronize()
        ee_ms = (time.perf_counter() - t2) * 1e3 / args.steps
        ee = (ee_ms, ee_n.cpu().numpy(), ee_t.cpu().numpy())
        log(f"[bench] early exit: {ee_ms:.4f} ms/step")
    # the statistics pass's reads alone (stage 3: same grid, chunks and loads,
    # no arithmetic) on the same inputs: the read rate that pass could reach
    ro = None
    if not tree and not args.early_exit and not small:
        ro_prep = [binding.spec_verify_sample_stage(3, tcopies[c], dcopies[c], tokens, uni, temps,
                                                    out_num_accepted=out_n, out_tokens=out_t, workspace=ws,
                                                    prepare=True) for c in range(R)]
        for k in range(min(args.warmup, 20)):
            ro_prep[k % R]()
        ro_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            ro_ev[k][0].record()
            ro_prep[k % R]()
            ro_ev[k][1].record()
        torch.cuda.synchronize()
        ro = np.array([e[0].elapsed_time(e[1]) for e in ro_ev])
        log(f"[bench] statistics reads alone: {ro.mean() * 1e3:.1f} us")
    per_kernel = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(ns)] for k in range(args.steps)])
    stage_ms = [float(v) for v in per_kernel.mean(axis=0)]
    log(f"[bench] {ms_per_step:.4f} ms/step; kernel event means (ms): {stage_ms}")

    def dist_us(v):
        return {"median": round(float(np.median(v)) * 1e3, 3), "p10": round(float(np.percentile(v, 10)) * 1e3, 3),
                "p90": round(float(np.percentile(v, 90)) * 1e3, 3)}

    detail = {"kernels": {n: {"mean_us": round(m * 1e3, 3), **{k + "_us": v for k, v in dist_us(per_kernel[:, i]).items()}}
                          for i, (n, m) in enumerate(zip(kernel_names, stage_ms))},
              "step_event_us": {**dist_us(per_kernel.sum(axis=1)), "steps": args.steps},
              "timing": "ms_per_step: wall clock over the timed steps (whole calls, nothing else on the stream); "
                        "kernel means and median/p10/p90: HIP events between the kernels in a second pass of as "
                        "many steps (step_event_us: per step, the sum of its kernels' event intervals)",
              "input_copies": R, "kernel_source_sha": sha}
    if tree:
        lens = outs[0].cpu().numpy()
        detail["mean_accept_len"] = float(lens[lens >= 0].mean())
        detail["invalid"] = int((lens < 0).sum())
        step_bytes = s1_bytes
    else:
        n_acc = out_n.cpu().numpy()
        _, s2_bytes = sample_bytes(inp.cfg, B, G, V, n_acc)
        step_bytes = s1_bytes + s2_bytes
        valid = n_acc >= 0
        detail["mean_accepted"] = float(n_acc[valid].mean())
        detail["mean_tokens_per_verify"] = float(n_acc[valid].mean() + 1)
        detail["invalid"] = int((~valid).sum())
        if args.early_exit:
            detail["one_pass_step_alg_bytes"] = int(s1_bytes + s2_bytes)
            s1_bytes = step_bytes = early_exit_bytes(inp.cfg, B, G, V, n_acc)
        elif small:
            s1_bytes = step_bytes  # one kernel reads the rows once and the draw row(s) again
        else:
            if ro is not None:
                detail["stats_reads_alone"] = {
                    "entry_point": "spec_verify_sample_stage(3)", "mean_us": round(float(ro.mean()) * 1e3, 3),
                    "median_us": round(float(np.median(ro)) * 1e3, 3),
                    "gbps": round(s1_bytes / (float(ro.mean()) * 1e-3) / 1e9, 1),
                    "stats_kernel_over_reads": round(stage_ms[0] / float(ro.mean()), 4),
                    "note": "the statistics kernel's grid, chunks and loads with its arithmetic replaced by an xor: "
                            "the rate at which it could read these bytes"}
            detail["kernels"]["sv_finish_kernel"]["alg_bytes"] = int(s2_bytes)
            detail["kernels"]["sv_finish_kernel"]["gbps"] = round(s2_bytes / (stage_ms[1] * 1e-3) / 1e9, 1)
    detail["kernels"][kernel_names[0]]["alg_bytes"] = int(s1_bytes)
    detail["kernels"][kernel_names[0]]["gbps"] = round(s1_bytes / (stage_ms[0] * 1e-3) / 1e9, 1)
    if ee is not None:
        ee_ms, ee_nacc, ee_tok = ee
        ee_bytes = early_exit_bytes(inp.cfg, B, G, V, ee_nacc)
        detail["early_exit"] = {
            "entry_point": "spec_verify_sample_early_exit", "ms_per_step": round(ee_ms, 5),
            "value": units / (ee_ms * 1e-3), "unit": unit, "alg_bytes": int(ee_bytes),
            "gbps": round(ee_bytes / (ee_ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(ee_bytes / (ee_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "same_outputs_as_one_pass": bool(np.array_equal(ee_nacc, n_acc) and
                                             np.array_equal(ee_tok, out_t.cpu().numpy()))}
    detail["step_alg_bytes"] = int(step_bytes)
    detail["step_gbps"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1)
    detail["step_frac_of_peak"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)

    achieved = s1_bytes / (stage_ms[0] * 1e-3) / 1e9
    line = {
        "metric": "verified draft positions/sec + achieved HBM GB/s (% peak), spec_verify at 1 GPU",
        "value": units / (ms_per_step * 1e-3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded logits standing in for target/draft model outputs",
        "config": cfg_desc,
        "roofline": {"bound": "hbm", "kernel": kernel_names[0], "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     # the profiled counters are per kernel of the one-pass path; the early-exit
                     # line spans several launches, which no single counter figure covers
                     "traffic": None if args.early_exit else traffic_from_profiles(args.workload, sha)},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
