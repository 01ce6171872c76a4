"""GPU tests of the draft-side sampler (spec_draft_sample) against the fp64
oracle: ragged multi-tile rows in both dtypes, the full-size draft workloads
of configurations 3 and 5 in the launch configuration the benchmark times,
masks and ties, invalid rows, strided rows, the staged entry point, and a
chi-square test of 10^6 draws."""
import numpy as np
import pytest
import torch
from scipy import stats

import synth
from oracle import spec_verify_oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _assert(t, name, allow_flags=2):
    H.log(f"[draft {name}] {t.summary()}")
    assert not t.fail, t.fail[:5]
    assert t.flagged <= max(allow_flags, 0.01 * t.checked)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("V,pad", [(1, 8), (7, 8), (33, 8), (4099, 8), (5000, None), (20000, None),
                                   (128257, 8)])
def test_rows_against_oracle(gpu, dt, V, pad):
    H.log(f"draft rows dt={dt} V={V} pad={pad}")
    d = synth.make_draft_rows(8, V, dt, T=[0.3, 0.7, 1.0, 1.0, 1.5, 2.0, 0.05, 10.0], seed=V)
    _assert(H.check_draft(d, H.run_draft(gpu, H.draft_tensors(d, pad_to=pad))), f"{dt} V={V}")


@pytest.mark.parametrize("cid", [3, 5])
def test_draft_workloads(gpu, cid):
    d = synth.make_draft_workload(cid, seed=0)
    H.log(f"draft workload of config {cid}: B={d.B} V={d.V} {d.dtype} (40 rows vs oracle)")
    out = H.run_draft(gpu, H.draft_tensors(d))
    rows = sorted(set(np.random.default_rng(cid).choice(d.B, 38, replace=False).tolist()) | {0, d.B - 1})
    _assert(H.check_draft(d, out, rows), f"config {cid}")
    assert (out["y"] >= 0).all()


@pytest.mark.parametrize("V", [3000, 2000])
def test_masks_ties_and_invalid(gpu, V):
    """V = 3000: the workgroup-per-row kernel; V = 2000 (one draw step): the
    wave-per-row kernel. The two-kernel (staged) path on the same rows too."""
    d = synth.make_draft_rows(10, V, "f32", T=1.0, seed=5)
    g = np.random.default_rng(5)
    L = d.logits
    L[0, g.random(V) < 0.9] = -np.inf          # mostly masked
    L[1, :] = 0.25                              # all ties
    L[2, :] = -np.inf
    L[2, V - 1] = 1.0                           # one token, at the end
    L[3, 17] = np.nan                           # invalid
    L[4, 5] = np.inf                            # invalid
    L[5, :] = -np.inf                           # invalid: no finite value
    d.temperature[6] = 0.0                      # invalid temperature
    d.uniforms[7] = 1.0                         # invalid uniform
    L[8, :V // 2] = -0.0
    L[8, V // 2:] = 0.0                         # signed zeros tie
    d.uniforms[9] = 0.0                         # u = 0: first token of positive mass
    tens = H.draft_tensors(d)
    for name, out in (("one pass", H.run_draft(gpu, tens)), ("staged", H.run_draft(gpu, tens, stage=True))):
        _assert(H.check_draft(d, out), f"masks/ties/invalid V={V} {name}")
        assert list(out["y"][3:8]) == [-1] * 5 and np.isnan(out["p"][3:8]).all()
        assert out["y"][2] == V - 1 and out["p"][2] == 1.0


def test_strided_rows_and_stages(gpu):
    d = synth.make_draft_rows(6, 3000, "bf16", T=0.9, seed=8)
    tens = H.draft_tensors(d)
    big = torch.full((6, 3064), float("nan"), dtype=torch.bfloat16, device="cuda")
    big[:, :3000] = tens["logits"]
    tens_s = dict(tens, logits=big[:, :3000])
    assert tens_s["logits"].stride() == (3064, 1)
    full = H.run_draft(gpu, tens)              # one-pass kernel (short rows)
    strided = H.run_draft(gpu, tens_s)
    staged = H.run_draft(gpu, tens_s, stage=True)  # the two-kernel path
    _assert(H.check_draft(d, strided), "strided")
    _assert(H.check_draft(d, staged), "staged")
    for k in full:
        assert np.array_equal(full[k].view(np.uint32), strided[k].view(np.uint32))


def test_chi_square_million_draws(gpu):
    """10^6 draws from one fixed row (10 calls of 10^5 rows at fresh uniforms)
    against q = softmax(L / T) computed by the oracle."""
    V, B, T = 32, 100000, 0.8
    L = np.random.default_rng(12).normal(0, 1.5, V).astype(np.float32)
    logits = torch.from_numpy(np.tile(L, (B, 1))).cuda()
    temps = torch.full((B,), T, dtype=torch.float32, device="cuda")
    g = np.random.default_rng(13)
    counts = np.zeros(V, np.int64)
    for _ in range(10):
        u = torch.from_numpy(synth.uniforms_u24(g, (B,))).cuda()
        y, _ = gpu.spec_draft_sample(logits, u, temps)
        counts += np.bincount(y.cpu().numpy(), minlength=V)
    q, _, _ = O.tempered_softmax(L.astype(np.float64), T)
    keep = q * counts.sum() >= 5
    obs, exp = counts[keep], q[keep] * counts.sum()
    if (~keep).any():  # pool the rare tokens into one bin
        obs, exp = np.append(obs, counts[~keep].sum()), np.append(exp, q[~keep].sum() * counts.sum())
    chi, p = stats.chisquare(obs, exp)
    H.log(f"[draft chi-square] 10^6 draws, V={V}: chi2={chi:.1f} p={p:.3f}")
    assert p > 1e-3


def test_bad_arguments_raise(gpu):
    d = synth.make_draft_rows(2, 100, "f32", seed=1)
    tens = H.draft_tensors(d)
    with pytest.raises(ValueError):
        gpu.spec_draft_sample(tens["logits"][:, :50].contiguous(), tens["uniforms"][:1], tens["temperature"])
    with pytest.raises(ValueError):
        gpu.spec_draft_sample(tens["logits"].double(), tens["uniforms"], tens["temperature"])


@pytest.mark.parametrize("T", [1e-6, 1e-12, 1e-30])
def test_temperature_extremes(gpu, T):
    d = synth.make_draft_rows(6, 3000, "bf16", T=T, seed=31)
    _assert(H.check_draft(d, H.run_draft(gpu, H.draft_tensors(d))), f"T={T}")


def test_huge_logits(gpu):
    """Logits around 10^8: the statistics pass takes its subtract form."""
    d = synth.make_draft_rows(6, 4000, "f32", T=[0.5, 1.0, 1.0, 2.0, 1.0, 0.7], seed=32, sd=2e7)
    _assert(H.check_draft(d, H.run_draft(gpu, H.draft_tensors(d))), "huge logits")


def test_both_paths_on_one_batch(gpu):
    """The one-pass kernel (B >= 128) and the two kernels (staged) on the same
    rows, each against the oracle."""
    d = synth.make_draft_rows(160, 70000, "bf16", T=0.9, seed=33)
    tens = H.draft_tensors(d)
    rows = list(range(0, 160, 8)) + [159]
    _assert(H.check_draft(d, H.run_draft(gpu, tens), rows), "one pass B=160")
    _assert(H.check_draft(d, H.run_draft(gpu, tens, stage=True), rows), "two kernels B=160")


def test_vocab_beyond_lds_steps(gpu):
    """V = 4.2M (2051 steps of 2048 tokens, beyond the kernels' LDS step
    arrays): the draft sampler's two-kernel path."""
    d = synth.make_draft_rows(2, 4_200_000, "f32", T=[0.8, 1.2], seed=34)
    _assert(H.check_draft(d, H.run_draft(gpu, H.draft_tensors(d))), "V=4.2M")
