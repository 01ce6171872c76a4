"""A sequence's result does not depend on its batch.

The statistics pass forms the same fp32 batches of every row however the call
splits the rows into chunks (chunks start on 16 KB batch boundaries; the chunk
size follows the call's total bytes, so it changes with B), and the finish
draws every sequence from the same per-step masses whether one or several
workgroups stream its draw row(s). Only fp64 additions of batch sums are
grouped differently, so the same sequences verified at B = 512, 64 and 1 (and
through the early-exit entry point, whose chunks are 128 KB) give the same
accept decisions and tokens, and diagnostics equal to fp64 rounding. The exact
result is what "Fast Inference from Transformers via Speculative Decoding"
asks of the method (abstract: identical outputs).
"""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _subset(tens, idx):
    ix = torch.as_tensor(idx, device=tens["target"].device)
    return {k: v.index_select(0, ix).contiguous() for k, v in tens.items()}


def _same(ref, out, idx, name, diag_rtol=1e-12):
    """out (a call on sequences idx) against rows idx of ref."""
    n_ref, n_out = ref["n"][idx], out["n"]
    assert np.array_equal(n_ref, n_out), (name, np.flatnonzero(n_ref != n_out)[:5])
    assert np.array_equal(ref["tokens"][idx], out["tokens"]), name
    for key in ("p_x", "q_x", "resid_mass"):
        a, b = ref[key][idx].astype(np.float64), out[key].astype(np.float64)
        both_nan = np.isnan(a) & np.isnan(b)
        ok = both_nan | (np.abs(a - b) <= diag_rtol * np.abs(a))
        assert ok.all(), (name, key, np.argwhere(~ok)[:3].tolist())


@pytest.mark.parametrize("cid", [5, 3])
def test_same_sequences_at_three_batch_sizes(gpu, cid):
    inp = synth.make_sample_inputs(cid, seed=0)
    tens = H.sample_tensors(inp)
    B = inp.B
    H.log(f"config {cid}: B={B} full batch, then 64 sequences, then single sequences")
    full = H.run_sample(gpu, tens)
    idx64 = np.arange(64) * (B // 64) + 3  # spread over the batch (every row class in config 5)
    sub = H.run_sample(gpu, _subset(tens, idx64))
    _same(full, sub, idx64, f"c{cid} B=64")
    for b in (0, 17, B // 2 + 1, B - 1):
        one = H.run_sample(gpu, _subset(tens, [b]))
        _same(full, one, np.array([b]), f"c{cid} B=1 seq {b}")
    # the early-exit entry point: 128 KB chunks, positions launched one group at a time
    ee = H.run_sample(gpu, tens, early_exit=True)
    assert np.array_equal(full["n"], ee["n"]) and np.array_equal(full["tokens"], ee["tokens"])
    ee64 = H.run_sample(gpu, _subset(tens, idx64), early_exit=True, tail_start=inp.gamma)
    assert np.array_equal(full["n"][idx64], ee64["n"]) and np.array_equal(full["tokens"][idx64], ee64["tokens"])
    H.log(f"[c{cid}] identical n and tokens at B={B}, 64, 1 and through early exit; "
          f"mean accepted {full['n'].mean():.3f}")


def test_small_vocab_batch_sizes(gpu):
    """V <= 2048: one wave per sequence, no chunking at all; B = 1 and B = 300 agree (rows of 1496 tokens: 16-byte aligned)."""
    inp = synth.make_custom_sample(300, 5, 1496, "bf16", "f32", T=0.8, noise_sd=0.6, seed=9)
    tens = H.sample_tensors(inp)
    full = H.run_sample(gpu, tens)
    for b in (0, 150, 299):
        _same(full, H.run_sample(gpu, _subset(tens, [b])), np.array([b]), f"V=1496 seq {b}", diag_rtol=0.0)
