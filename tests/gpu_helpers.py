"""Shared code of the GPU tests: upload inputs, call the C ABI through the
binding, and check results against the fp64 oracle with the parity contract.

Parity contract (sampling):
  * accept decisions equal at every position both sides reached; a differing
    decision is excused (flagged) only when |u_i - rho_i| < 1e-6 with the
    oracle's rho, and then the rest of the sequence is excused;
  * the final token equal; a different token is excused (flagged) only when
    u_gamma lies within 1e-6 of the oracle's CDF interval of the GPU's token;
  * p(x), q(x) and the drawn distribution's mass within 1e-5 relative;
  * invalid sequences (-1) agree exactly.
Tree results are compared bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import spec_verify_oracle as O

FLAG_WINDOW = 1e-6
PROB_RTOL = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_logits(a: np.ndarray, dt: str, device="cuda") -> torch.Tensor:
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def padded_logits(a: np.ndarray, dt: str, pad_to: int, device="cuda") -> torch.Tensor:
    """Upload [..][V] logits into rows of a multiple-of-`pad_to` stride; returns the [..., :V] view."""
    V = a.shape[-1]
    Vp = -(-V // pad_to) * pad_to
    # NaN padding: the kernels must mask everything past V in a row's last 16-byte block
    fill = np.uint16(0x7FC1) if dt == "bf16" else np.float32(np.nan)
    big = np.full(a.shape[:-1] + (Vp,), fill, dtype=a.dtype)
    big[..., :V] = a
    return dev_logits(big, dt, device)[..., :V]


def sample_tensors(inp, device="cuda", pad_to=None):
    cfg = inp.cfg
    tdt, ddt = cfg.target_dtype, cfg.draft_dtype
    if pad_to:
        t = padded_logits(inp.target, tdt, pad_to, device)
        d = padded_logits(inp.draft, ddt, pad_to, device)
    else:
        t = dev_logits(inp.target, tdt, device)
        d = dev_logits(inp.draft, ddt, device)
    B = inp.tokens.shape[0]
    if t.shape[0] != B:  # shared logits: stride-0 batch dimension
        t = t.expand(B, *t.shape[1:])
        d = d.expand(B, *d.shape[1:])
    return dict(target=t, draft=d, draft_tokens=torch.from_numpy(inp.tokens).to(device),
                uniforms=torch.from_numpy(inp.uniforms).to(device),
                temperature=torch.from_numpy(inp.temperature).to(device))


def run_sample(binding, tens, diag=True, workspace=None, early_exit=False, tail_start=None):
    """early_exit: the early-exit entry point; tail_start (with early_exit) the
    grouped one with that grouping of positions."""
    if early_exit and tail_start is not None:
        n, tok, d = binding.spec_verify_sample_early_exit_grouped(tail_start, **tens, diag=diag, workspace=workspace)
    else:
        fn = binding.spec_verify_sample_early_exit if early_exit else binding.spec_verify_sample
        n, tok, d = fn(**tens, diag=diag, workspace=workspace)
    torch.cuda.synchronize()
    out = {"n": n.cpu().numpy(), "tokens": tok.cpu().numpy()}
    if d:
        out.update({k: v.cpu().numpy() for k, v in d.items()})
    return out


def run_sample_staged(binding, tens, workspace=None):
    """The two kernels of spec_verify_sample called one stage at a time (the
    statistics pass, then the finish), whatever the vocabulary size."""
    ws = workspace if workspace is not None else binding.Workspace()
    n, tok, _ = binding.spec_verify_sample_stage(1, **tens, workspace=ws)
    n, tok, d = binding.spec_verify_sample_stage(2, **tens, out_num_accepted=n, out_tokens=tok, diag=True,
                                                 workspace=ws)
    torch.cuda.synchronize()
    out = {"n": n.cpu().numpy(), "tokens": tok.cpu().numpy()}
    out.update({k: v.cpu().numpy() for k, v in d.items()})
    return out


def compare_one_pass(one, ee):
    """Early exit against the one-pass call on the same inputs. Returns
    (differing, bad): the sequences whose n or tokens differ (both results are
    checked against the oracle by the caller), and a list of other problems:
    for sequences that agree and are valid, p(x), q(x) of positions 0..n and
    the drawn distribution's mass must agree within PROB_RTOL, and p(x), q(x)
    of every position the early-exit call reports after n must be NaN or equal
    to the one-pass value within PROB_RTOL (tail-group rows are read)."""
    differ = np.flatnonzero((one["n"] != ee["n"]) | (one["tokens"] != ee["tokens"]).any(axis=1))
    bad = []
    if "p_x" in one and "p_x" in ee:
        B, G = one["p_x"].shape
        for b in range(B):
            n = int(one["n"][b])
            if n < 0 or b in differ:
                continue
            for key in ("p_x", "q_x"):
                for i in range(G):
                    o, e = float(one[key][b, i]), float(ee[key][b, i])
                    if i > n and np.isnan(e):
                        continue
                    if not (np.isfinite(o) and np.isfinite(e) and _rel(e, o) <= PROB_RTOL):
                        bad.append((key, b, i, o, e))
            if _rel(ee["resid_mass"][b], one["resid_mass"][b]) > PROB_RTOL:
                bad.append(("resid_mass", b))
    return differ, bad


class Tally:
    def __init__(self):
        self.checked = 0
        self.flag_accept = 0
        self.flag_draw = 0
        self.fail = []
        self.max_prob_rel = 0.0
        self.max_mass_rel = 0.0

    @property
    def flagged(self):
        return self.flag_accept + self.flag_draw

    def summary(self):
        return (f"checked={self.checked} flagged(accept={self.flag_accept}, draw={self.flag_draw}) "
                f"unflagged_mismatches={len(self.fail)} max_prob_rel={self.max_prob_rel:.3g}")


def _rel(a, b):
    a, b = float(a), float(b)
    if abs(b) < 1e-30:
        return 0.0 if abs(a) < 1e-30 else float("inf")
    return abs(a - b) / abs(b)


def check_sample_seq(tally: Tally, b: int, Lt, Ld, x, u, T, gpu, lb=None):
    """Check sequence b of a GPU result against the oracle (Lt, Ld already float64)."""
    o = O.verify_sample_sequence(Lt, Ld, x, u, T, keep_cdf=True)
    tally.checked += 1
    gn = int(gpu["n"][b])
    gt = [int(v) for v in gpu["tokens"][b]]
    G = len(x)
    if not o.valid:
        if gn != -1 or any(v != -1 for v in gt):
            tally.fail.append((b, "oracle invalid, gpu valid", gn))
        return o
    if gn < 0:
        tally.fail.append((b, "gpu invalid, oracle valid", o.n))
        return o
    if gn != o.n:
        i = min(gn, o.n)
        if abs(float(u[i]) - float(o.rho[i])) < FLAG_WINDOW:
            tally.flag_accept += 1
            return o
        tally.fail.append((b, "accept decision", i, gn, o.n, float(u[i]), float(o.rho[i])))
        return o
    n = gn
    if gt[:n] != [int(v) for v in x[:n]]:
        tally.fail.append((b, "accepted tokens", gt[:n]))
        return o
    if any(v != -1 for v in gt[n + 1:]):
        tally.fail.append((b, "padding", gt))
        return o
    y = gt[n]
    if y != o.y:
        cdf = o.cdf
        if not (0 <= y < len(cdf)):
            tally.fail.append((b, "token out of range", y))
            return o
        lo = cdf[y - 1] if y > 0 else 0.0
        hi = cdf[y]
        uu = float(u[G])
        dist = 0.0 if lo <= uu < hi else min(abs(uu - lo), abs(uu - hi))
        if dist < FLAG_WINDOW:
            tally.flag_draw += 1
        else:
            tally.fail.append((b, "draw", y, o.y, uu, lo, hi))
        return o
    # probabilities
    if "p_x" in gpu:
        # a NaN (or inf) diagnostic of a valid sequence fails: _rel is then NaN
        # or inf, and only a finite value within the tolerance passes
        for i in range(min(n + 1, G)):
            for key, ref in (("p_x", o.p_x[i]), ("q_x", o.q_x[i])):
                g = float(gpu[key][b, i])
                if float(ref) >= 1e-30 or not (g < 1e-30):
                    r = _rel(g, ref)
                    if np.isfinite(r):
                        tally.max_prob_rel = max(tally.max_prob_rel, r)
                    if not (np.isfinite(g) and r <= PROB_RTOL):
                        tally.fail.append((b, key, i, g, float(ref)))
        g = float(gpu["resid_mass"][b])
        r = _rel(g, o.resid_mass)
        if np.isfinite(r):
            tally.max_prob_rel = max(tally.max_prob_rel, r)
            tally.max_mass_rel = max(tally.max_mass_rel, r)
        if not (np.isfinite(g) and r <= PROB_RTOL) and not o.fallback:
            tally.fail.append((b, "resid_mass", g, o.resid_mass))
    return o


def check_sample_parallel(inp, gpu, seqs=None, workers=16):
    """check_sample over threads (numpy releases the GIL in the oracle's array
    work); the tallies of the threads are merged in sequence order."""
    from concurrent.futures import ThreadPoolExecutor
    B = inp.tokens.shape[0]
    seqs = list(range(B)) if seqs is None else list(seqs)
    parts = [seqs[i::workers] for i in range(workers)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        tallies = list(ex.map(lambda part: check_sample(inp, gpu, part), [p for p in parts if p]))
    out = Tally()
    for t in tallies:
        out.checked += t.checked
        out.flag_accept += t.flag_accept
        out.flag_draw += t.flag_draw
        out.fail += t.fail
        out.max_prob_rel = max(out.max_prob_rel, t.max_prob_rel)
        out.max_mass_rel = max(out.max_mass_rel, t.max_mass_rel)
    return out


def check_sample(inp, gpu, seqs=None, tally=None):
    tally = tally or Tally()
    cfg = inp.cfg
    B = inp.tokens.shape[0]
    seqs = range(B) if seqs is None else seqs
    shared = inp.target.shape[0] != B
    cache = {}
    for b in seqs:
        lb = 0 if shared else b
        if lb not in cache:
            cache = {lb: (O.widen(inp.target[lb], cfg.target_dtype), O.widen(inp.draft[lb], cfg.draft_dtype))}
        Lt, Ld = cache[lb]
        check_sample_seq(tally, b, Lt, Ld, inp.tokens[b], inp.uniforms[b].astype(np.float64),
                         float(inp.temperature[b]), gpu)
    return tally


# ---------------------------------------------------------------------------
# tree
# ---------------------------------------------------------------------------
def tree_tensors(ti, device="cuda", dtype=None):
    dt = dtype or ti.dtype
    return dict(logits=dev_logits(ti.logits, dt, device), parents=torch.from_numpy(ti.parents).to(device),
                tokens=torch.from_numpy(ti.tokens).to(device))


def run_tree(binding, tens, workspace=None):
    L, P, Bn, A = binding.spec_verify_greedy_tree(**tens, workspace=workspace)
    torch.cuda.synchronize()
    return {"len": L.cpu().numpy(), "path": P.cpu().numpy(), "bonus": Bn.cpu().numpy(), "argmax": A.cpu().numpy()}


def check_tree(logits_np, dt, parents, tokens, gpu, seqs=None):
    fails = []
    B, N = parents.shape
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        o = O.verify_tree_sequence(O.widen(logits_np[b], dt), parents[b], tokens[b])
        want_arg = [int(v) for v in o.argmax]
        got_arg = [int(v) for v in gpu["argmax"][b]]
        if want_arg != got_arg:
            fails.append((b, "argmax", [(j, got_arg[j], want_arg[j]) for j in range(N) if got_arg[j] != want_arg[j]][:5]))
        if not o.valid:
            if gpu["len"][b] != -1 or gpu["bonus"][b] != -1 or (gpu["path"][b] != -1).any():
                fails.append((b, "invalid tree reported valid"))
            continue
        path = [int(v) for v in gpu["path"][b]]
        want_path = o.path + [-1] * (N - len(o.path))
        if int(gpu["len"][b]) != o.accept_len or path != want_path or int(gpu["bonus"][b]) != o.bonus:
            fails.append((b, "tree", int(gpu["len"][b]), o.accept_len, int(gpu["bonus"][b]), o.bonus, path[:8],
                          want_path[:8]))
    return fails


# ---------------------------------------------------------------------------
# draft-side sampler
# ---------------------------------------------------------------------------
def draft_tensors(d, device="cuda", pad_to=None):
    t = padded_logits(d.logits, d.dtype, pad_to, device) if pad_to else dev_logits(d.logits, d.dtype, device)
    return dict(logits=t, uniforms=torch.from_numpy(d.uniforms).to(device),
                temperature=torch.from_numpy(d.temperature).to(device))


def run_draft(binding, tens, workspace=None, stage=None):
    if stage is None:
        y, p = binding.spec_draft_sample(**tens, want_prob=True, workspace=workspace)
    else:
        y = p = None
        for s in (1, 2):
            y, p = binding.spec_draft_sample(**tens, want_prob=True, workspace=workspace, stage=s,
                                             out_tokens=y)
    torch.cuda.synchronize()
    return {"y": y.cpu().numpy(), "p": p.cpu().numpy()}


def check_draft(d, gpu, rows=None, tally=None):
    """Check draft-sampler outputs against the oracle: the token equal, or u
    within FLAG_WINDOW of the oracle's CDF interval of the GPU's token
    (flagged); q(token) within PROB_RTOL; invalid rows -1 exactly."""
    tally = tally or Tally()
    rows = range(d.B) if rows is None else rows
    for b in rows:
        L = O.widen(d.logits[b], d.dtype)
        u = float(d.uniforms[b])
        o = O.draft_sample_row(L, float(d.temperature[b]), u, keep_cdf=True)
        tally.checked += 1
        gy, gp = int(gpu["y"][b]), float(gpu["p"][b])
        if not o.valid:
            if gy != -1 or not np.isnan(gp):
                tally.fail.append((b, "oracle invalid, gpu valid", gy))
            continue
        if gy != o.y:
            if not (0 <= gy < len(o.cdf)):
                tally.fail.append((b, "token out of range", gy))
                continue
            lo = o.cdf[gy - 1] if gy > 0 else 0.0
            hi = o.cdf[gy]
            dist = 0.0 if lo <= u < hi else min(abs(u - lo), abs(u - hi))
            if dist < FLAG_WINDOW:
                tally.flag_draw += 1
            else:
                tally.fail.append((b, "draw", gy, o.y, u, lo, hi))
            continue
        r = _rel(gp, o.q_y)
        tally.max_prob_rel = max(tally.max_prob_rel, r)
        if r > PROB_RTOL:
            tally.fail.append((b, "q_y", gp, o.q_y))
    return tally
