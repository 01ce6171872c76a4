"""Calibrate the draft-noise scale of sampling configs 2, 3 and 5.

Writes synth/draft_noise.json, the only stored value the input generators read.
It calls the fp64 oracle (tempered_softmax, alpha) and the seeded generators;
nothing else. Run from the repository root:

    python -m oracle.calibrate_draft_noise

For each config the draft is the rounded target plus N(0, s) noise (config 5:
s = c * T_b on its "normal" rows), and s (or c) is found by bisection so that
the mean overlap alpha = sum_v min(p_v, q_v) over a 16-row subsample equals
the config's goal (0.70, 0.60, 0.70). The subsample uses common random numbers:
the same target rows and the same standard-normal noise at every trial value,
so alpha is monotone in s and the bisection is exact up to its tolerance.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synth  # noqa: E402
from oracle.spec_verify_oracle import alpha, tempered_softmax  # noqa: E402


def subsample_rows(cid: int, seed: int = 0, nrows: int = 16):
    """(target_rows_f64, noise_z_f32, T, draft_dtype) for a 16-row subsample."""
    cfg = synth.CONFIGS[cid]
    bias = synth.zipf_bias(seed, cfg.V) if cid == 2 else None
    cls = synth.row_classes(cfg, seed)
    temps = synth.temperatures(cfg, seed, cfg.B)
    rows, zs, Ts = [], [], []
    b = 0
    while len(rows) < nrows:
        if cls[b] != 0:
            b += 1
            continue
        t32 = synth.target_rows(cfg, seed, b, cfg.gamma + 1, bias)
        t_round = synth.decode(synth._to_dtype(t32, cfg.target_dtype), cfg.target_dtype)
        z = synth.gen(seed, cid, synth.S_DRAFT, b).standard_normal((cfg.gamma, cfg.V), dtype=np.float32)
        for i in range(cfg.gamma):
            if len(rows) < nrows:
                rows.append(t_round[i])
                zs.append(z[i])
                Ts.append(float(temps[b]))
        b += 1
    return rows, zs, Ts, cfg


def mean_alpha(rows, zs, Ts, cfg, s: float) -> float:
    vals = []
    for t, z, T in zip(rows, zs, Ts):
        sd = s * T if cfg.cid == 5 else s
        d32 = t + z * np.float32(sd)
        dq = synth.decode(synth._to_dtype(d32, cfg.draft_dtype), cfg.draft_dtype).astype(np.float64)
        p, _, _ = tempered_softmax(t.astype(np.float64), T)
        q, _, _ = tempered_softmax(dq, T)
        vals.append(alpha(p, q))
    return float(np.mean(vals))


def calibrate(cid: int, seed: int = 0, tol: float = 1e-4):
    rows, zs, Ts, cfg = subsample_rows(cid, seed)
    goal = cfg.alpha_goal
    lo, hi = 0.0, 8.0
    a_hi = mean_alpha(rows, zs, Ts, cfg, hi)
    assert a_hi < goal, (cid, a_hi)
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        a = mean_alpha(rows, zs, Ts, cfg, mid)
        if a > goal:
            lo = mid
        else:
            hi = mid
        if hi - lo < tol:
            break
    s = 0.5 * (lo + hi)
    return {"scale": s, "alpha_goal": goal, "alpha_subsample": mean_alpha(rows, zs, Ts, cfg, s),
            "meaning": "draft noise sd (config 5: sd = scale * T_b on normal rows)",
            "subsample": "16 rows, seed 0, common random numbers"}


def main():
    out = {}
    for cid in (2, 3, 5):
        out[str(cid)] = calibrate(cid)
        print(cid, out[str(cid)], flush=True)
    out["written_by"] = "oracle/calibrate_draft_noise.py"
    with open(synth.CALIBRATION_FILE, "w") as f:
        json.dump(out, f, indent=2, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
