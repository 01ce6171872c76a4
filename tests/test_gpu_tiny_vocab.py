"""GPU tests of the sampling verify at tiny vocabularies (V <= 32 with
2 gamma + 1 <= 32 rows: two sequences per wave) against the fp64 oracle and
the two-kernel (staged) path: both halves of a wave, a half past the batch
(odd B), gamma at the boundary of the two-per-wave form (15) and just past it
(16, one sequence per wave), every dtype pair, masks and signed zeros,
identical and disjoint rows, invalid inputs, unconsulted positions, and the
draft sampler's rows of at most 32 tokens."""
import numpy as np
import pytest

import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _check(inp, out, name, allow_flags=2):
    t = H.check_sample(inp, out)
    H.log(f"[tiny {name}] {t.summary()}")
    assert not t.fail, t.fail[:5]
    assert t.flagged <= allow_flags
    return t


def _full_and_staged(gpu, inp, name, pad=8):
    tens = H.sample_tensors(inp, pad_to=pad)
    out = H.run_sample(gpu, tens)
    _check(inp, out, name)
    _check(inp, H.run_sample_staged(gpu, tens), name + " staged")
    return out


@pytest.mark.parametrize("tdt,ddt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("B,G,V", [(1, 1, 1), (2, 1, 2), (7, 3, 17), (9, 4, 32), (5, 15, 32), (3, 15, 5),
                                   (5, 16, 32), (4, 7, 31)])
def test_shapes_and_dtypes(gpu, tdt, ddt, B, G, V):
    H.log(f"tiny vocab B={B} gamma={G} V={V} {tdt}/{ddt}")
    T = np.linspace(0.5, 1.6, B, dtype=np.float32)
    inp = synth.make_custom_sample(B, G, V, tdt, ddt, T=T, noise_sd=0.7, seed=1000 * G + V + B)
    out = _full_and_staged(gpu, inp, f"B={B} G={G} V={V} {tdt}/{ddt}")
    assert (out["n"] >= 0).all()


def test_full_acceptance_at_the_boundary(gpu):
    """Drafts equal to the target at gamma = 15: every draft accepted, the
    bonus token drawn from row 15."""
    inp = synth.make_custom_sample(7, 15, 32, "f32", "f32", T=1.0, seed=7)
    inp.draft[:] = inp.target[:, :15]
    out = _full_and_staged(gpu, inp, "gamma 15 identical")
    assert (out["n"] == 15).all()


def test_masks_signed_zero_identical_disjoint(gpu):
    """-inf masks, -0 / +0 logits, identical rows (sequences 0-2) and
    disjoint supports at position 0 (sequences 3-5) at V = 32."""
    V = 32
    inp = synth.make_custom_sample(11, 4, V, "bf16", "bf16", T=1.0, seed=21)
    g = np.random.default_rng(21)
    ninf = synth.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    mz = synth.f32_to_bf16_bits(np.array([-0.0], np.float32))[0]
    for arr in (inp.target[6:], inp.draft[6:]):
        arr[g.random(arr.shape) < 0.3] = ninf
        arr[g.random(arr.shape) < 0.05] = mz
        arr[g.random(arr.shape) < 0.05] = 0
    for b in range(6, 11):
        for i in range(4):
            inp.draft[b, i, inp.tokens[b, i]] = 0
    inp.draft[:3] = inp.target[:3, :4]
    for b in range(3, 6):
        inp.target[b, 0, 16:] = ninf
        inp.draft[b, 0, :16] = ninf
        inp.tokens[b, 0] = 16 + (b * 5) % 16
    out = _full_and_staged(gpu, inp, "masks / identical / disjoint")
    assert (out["n"][:3] == 4).all() and (out["n"][3:6] == 0).all()
    assert (out["tokens"][3:6, 0] < 16).all()


def test_invalid_inputs(gpu):
    """Every sequence invalid at a position the method consults (both halves
    of a wave, and a valid neighbour beside an invalid one)."""
    V = 32
    inp = synth.make_custom_sample(13, 4, V, "f32", "f32", T=1.0, seed=5)
    T = inp.temperature
    T[0], T[1], T[2], T[3], T[4] = 0.0, -1.0, np.nan, np.inf, 1e-40
    inp.tokens[5, 0] = V
    inp.tokens[6, 0] = -1
    inp.target[7, 0, 17] = np.nan
    inp.draft[8, 0, 3] = np.inf
    inp.target[9, 0, :] = -np.inf
    inp.uniforms[10, 0] = 1.0
    inp.uniforms[11, 4] = -0.5
    out = _full_and_staged(gpu, inp, "invalid")
    assert (out["n"][:12] == -1).all() and (out["tokens"][:12] == -1).all()
    assert out["n"][12] >= 0


def test_unconsulted_positions(gpu):
    """A rejection at position 0 followed by a bad token, NaN rows and a bad
    uniform the method never consults: every sequence valid."""
    V = 24
    inp = synth.make_custom_sample(5, 5, V, "f32", "f32", T=1.0, seed=6)
    for b in range(5):
        inp.target[b, 0, 12:] = -np.inf
        inp.draft[b, 0, :12] = -np.inf
        inp.tokens[b, 0] = 14
    inp.tokens[0, 2] = 9999
    inp.target[1, 3, 5] = np.nan
    inp.draft[2, 1, :] = np.nan
    inp.uniforms[3, 2] = 7.0
    out = _full_and_staged(gpu, inp, "unconsulted")
    assert (out["n"] == 0).all() and (out["tokens"][:, 0] < 12).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,V", [(1, 1), (9, 32), (64, 20)])
def test_draft_sampler_rows(gpu, dt, B, V):
    """spec_draft_sample on rows of at most 32 tokens (gamma = 0 in the
    two-per-wave kernel), against the oracle and the staged path."""
    T = np.linspace(0.4, 2.0, B, dtype=np.float32)
    d = synth.make_draft_rows(B, V, dt, T=T, seed=B + V)
    tens = H.draft_tensors(d, pad_to=8)
    for name, out in (("one pass", H.run_draft(gpu, tens)), ("staged", H.run_draft(gpu, tens, stage=True))):
        t = H.check_draft(d, out)
        H.log(f"[tiny draft B={B} V={V} {dt} {name}] {t.summary()}")
        assert not t.fail, t.fail[:5]
        assert t.flagged <= 2
