"""GPU parity: the HIP path against the fp64 oracle, element by element on small
multi-tile cases and on the five full-size workloads in the launch
configuration the benchmark times: every sequence at the benchmark's seed 0,
and sampled sequences at seeds 1 and 2."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _assert_tally(t, name, max_flag_frac=0.01):
    H.log(f"[{name}] {t.summary()} max_mass_rel={t.max_mass_rel:.3g}")
    assert not t.fail, t.fail[:5]
    assert t.flagged <= max(2, max_flag_frac * t.checked), t.summary()


@pytest.mark.parametrize("tdt,ddt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("V,pad", [(5000, None), (4099, 8), (20000, None)])
def test_small_multitile(gpu, tdt, ddt, V, pad):
    H.log(f"small multitile tdt={tdt} ddt={ddt} V={V} pad={pad}")
    inp = synth.make_custom_sample(6, 3, V, tdt, ddt, T=[0.5, 0.9, 1.0, 1.3, 2.0, 0.7], noise_sd=0.8, seed=V)
    out = H.run_sample(gpu, H.sample_tensors(inp, pad_to=pad))
    _assert_tally(H.check_sample(inp, out), f"small {tdt}/{ddt} V={V}")


def test_config1_tiny(gpu):
    H.log("config 1: B=1 x 10^4 trials, gamma=4, V=32, fp32, shared logits (stride 0)")
    inp = synth.make_sample_inputs(1, seed=0)
    out = H.run_sample(gpu, H.sample_tensors(inp))
    _assert_tally(H.check_sample(inp, out), "config1")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config2(gpu, seed):
    H.log(f"config 2: B=64 gamma=4 V=32000 bf16, seed {seed}")
    inp = synth.make_sample_inputs(2, seed=seed)
    out = H.run_sample(gpu, H.sample_tensors(inp))
    _assert_tally(H.check_sample(inp, out), f"config2 seed {seed}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config3(gpu, seed):
    """Seed 0: all 256 sequences; seeds 1, 2: 48 sampled sequences."""
    H.log(f"config 3: B=256 gamma=8 V=128256 bf16 T=0.7, seed {seed}")
    inp = synth.make_sample_inputs(3, seed=seed)
    out = H.run_sample(gpu, H.sample_tensors(inp))
    if seed == 0:
        seqs = list(range(inp.B))
    else:
        seqs = sorted(set(np.random.default_rng(3 + 100 * seed).choice(inp.B, 46, replace=False).tolist())
                      | {0, inp.B - 1})
    t = H.check_sample_parallel(inp, out, seqs)
    _assert_tally(t, f"config3 seed {seed}")
    assert t.checked == len(seqs)
    assert (out["n"] >= 0).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config5(gpu, seed):
    """Seed 0: all 512 sequences; seeds 1, 2: 16 sampled sequences of each row class."""
    H.log(f"config 5: B=512 gamma=5 V=256000 bf16 target / fp32 draft, per-row T, seed {seed}")
    inp = synth.make_sample_inputs(5, seed=seed)
    out = H.run_sample(gpu, H.sample_tensors(inp))
    if seed == 0:
        seqs = list(range(inp.B))
    else:
        rng = np.random.default_rng(5 + 100 * seed)
        seqs = []
        for cls in (0, 1, 2):
            idx = np.flatnonzero(inp.row_class == cls)
            seqs += rng.choice(idx, 16, replace=False).tolist()
        seqs = sorted(seqs)
    t = H.check_sample_parallel(inp, out, seqs)
    _assert_tally(t, f"config5 seed {seed}")
    assert t.checked == len(seqs)
    # class properties on every sequence: identical rows accept all drafts, disjoint rows reject at once
    assert (out["n"][inp.row_class == 2] == inp.gamma).all()
    assert (out["n"][inp.row_class == 1] == 0).mean() > 0.99


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config4_tree(gpu, seed):
    H.log(f"config 4: 32 trees x 60 nodes, V=32000 bf16, seed {seed}")
    ti = synth.make_tree_inputs(4, seed=seed)
    out = H.run_tree(gpu, H.tree_tensors(ti))
    fails = H.check_tree(ti.logits, "bf16", ti.parents, ti.tokens, out)
    H.log(f"[config4] trees={ti.parents.shape[0]} mismatches={len(fails)} mean_len={out['len'].mean():.2f}")
    assert not fails, fails[:3]


def test_tree_fp32_and_multichunk(gpu):
    H.log("tree fp32, V=300000 (several chunks per row), B=3 N=17")
    ti = synth.make_tree_inputs(4, seed=7, B=3, N=17, V=300000, dtype="f32")
    out = H.run_tree(gpu, H.tree_tensors(ti))
    fails = H.check_tree(ti.logits, ti.dtype, ti.parents, ti.tokens, out)
    assert not fails, fails[:3]


def test_repeat_calls_are_bit_identical(gpu):
    H.log("determinism: config 2 twice, tree twice")
    inp = synth.make_sample_inputs(2, seed=1)
    tens = H.sample_tensors(inp)
    a = H.run_sample(gpu, tens)
    b = H.run_sample(gpu, tens)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    ti = synth.make_tree_inputs(4, seed=1)
    tt = H.tree_tensors(ti)
    x, y = H.run_tree(gpu, tt), H.run_tree(gpu, tt)
    for k in x:
        assert np.array_equal(x[k], y[k]), k
