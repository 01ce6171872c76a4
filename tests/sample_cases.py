"""Seeded sampling-verify edge cases shared by the GPU tests of both entry
points (one pass and early exit). Builders only: no verify arithmetic."""
from __future__ import annotations

import numpy as np

import synth


def custom(B=6, G=4, V=1024, tdt="f32", ddt="f32", seed=0):
    return synth.make_custom_sample(B, G, V, tdt, ddt, T=1.0, seed=seed)


def masks_and_signed_zero():
    """30% -inf masks, -0 and +0 logits; every draft token stays drawable."""
    inp = custom(8, 4, 1000, "bf16", "bf16", seed=2)
    g = np.random.default_rng(2)
    ninf = synth.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    mz = synth.f32_to_bf16_bits(np.array([-0.0], np.float32))[0]
    for arr in (inp.target, inp.draft):
        m = g.random(arr.shape) < 0.3
        arr[m] = ninf
        arr[g.random(arr.shape) < 0.05] = mz
        arr[g.random(arr.shape) < 0.05] = 0
    for b in range(inp.B):
        for i in range(inp.gamma):
            inp.draft[b, i, inp.tokens[b, i]] = 0
    return inp


def identical_and_disjoint():
    """Sequences 0-3: draft rows equal to the target's (accept all); 4-7:
    disjoint supports at position 0 (reject at once, draw below 1500)."""
    inp = custom(8, 5, 3000, "bf16", "bf16", seed=4)
    inp.draft[:4] = inp.target[:4, :5]
    ninf = synth.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    for b in range(4, 8):
        inp.target[b, 0, 1500:] = ninf
        inp.draft[b, 0, :1500] = ninf
        inp.tokens[b, 0] = 1500 + (b * 37) % 1500
    return inp


def invalid_inputs():
    """Every sequence is invalid at a position the method consults."""
    inp = custom(12, 4, 512, "f32", "f32", seed=5)
    T = inp.temperature
    T[0], T[1], T[2], T[3], T[4] = 0.0, -1.0, np.nan, np.inf, 1e-40
    inp.tokens[5, 0] = 512
    inp.tokens[6, 0] = -1
    inp.target[7, 0, 17] = np.nan
    inp.draft[8, 0, 3] = np.inf
    inp.target[9, 0, :] = -np.inf
    inp.uniforms[10, 0] = 1.0
    inp.uniforms[11, 4] = -0.5
    return inp


def unconsulted_positions():
    """A rejection at position 0 (disjoint supports) followed by bad tokens,
    NaN rows and a bad uniform that the method never consults."""
    inp = custom(4, 5, 700, "f32", "f32", seed=6)
    for b in range(4):
        inp.target[b, 0, 350:] = -np.inf
        inp.draft[b, 0, :350] = -np.inf
        inp.tokens[b, 0] = 400
    inp.tokens[0, 2] = 9999
    inp.target[1, 3, 5] = np.nan
    inp.draft[2, 1, :] = np.nan
    inp.uniforms[3, 2] = 7.0
    return inp


def invalid_after_accepts():
    """Invalid data at a later position that is reached (draft rows equal to
    the target's, so every earlier draft is accepted): NaN in target row 2 of
    sequence 0, an out-of-range token at position 3 of sequence 1, a bad bonus
    row of sequence 2 (all reached), and NaN in row 2 of sequence 3 after a
    rejection at position 1 (not reached: valid)."""
    inp = custom(4, 4, 900, "f32", "f32", seed=11)
    inp.draft[:] = inp.target[:, :4]
    inp.target[0, 2, 100] = np.nan
    inp.tokens[1, 3] = 900
    inp.target[2, 4, :] = -np.inf
    inp.target[3, 1, 450:] = -np.inf
    inp.draft[3, 1, :450] = -np.inf
    inp.tokens[3, 1] = 600
    inp.target[3, 2, 7] = np.nan
    return inp
