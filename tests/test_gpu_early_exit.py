"""GPU tests of the early-exit sampling verify (rows after a sequence's first
rejection are never read): against the fp64 oracle with the parity contract,
and against the one-pass entry point on the same inputs (same outputs bit for
bit). Small multi-tile cases, the full-size workloads in the launch
configuration the benchmark times, extreme gamma and the edge cases."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_helpers as H
from tests import sample_cases as SC

pytestmark = pytest.mark.gpu


# Groupings of positions: chosen from the sizes (small cases get one launch
# with no gate), position 0 alone and then the rest, every position gated.
GROUPINGS = ["auto", "first", "all"]


def _tail_start(grouping, inp):
    return {"auto": None, "first": 1, "all": int(inp.tokens.shape[1])}[grouping]


def _both(gpu, inp, pad=None, seqs=None, name="", allow_flags=2, workspace=None, grouping="auto"):
    """Early exit against the oracle (on `seqs`, default all) and against the
    one-pass call; a sequence where the two calls differ must be within the
    parity contract (a flagged case) for both of them."""
    tens = H.sample_tensors(inp, pad_to=pad)
    one = H.run_sample(gpu, tens, workspace=workspace)
    ee = H.run_sample(gpu, tens, workspace=workspace, early_exit=True, tail_start=_tail_start(grouping, inp))
    name = f"{name} ({grouping})"
    differ, bad = H.compare_one_pass(one, ee)
    assert not bad, (name, bad[:5])
    B = inp.tokens.shape[0]
    check = sorted(set(range(B) if seqs is None else seqs) | set(differ.tolist()))
    t = H.check_sample(inp, ee, check)
    t1 = H.check_sample(inp, one, differ.tolist())
    H.log(f"[early exit {name}] {t.summary()}; differs from one pass on {len(differ)} "
          f"(one pass there: {t1.summary()})")
    assert not t.fail and not t1.fail, (t.fail[:3], t1.fail[:3])
    assert t.flagged <= max(allow_flags, 0.01 * t.checked)
    assert len(differ) <= t.flagged + t1.flagged
    return ee


@pytest.mark.parametrize("grouping", GROUPINGS)
@pytest.mark.parametrize("tdt,ddt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("V,pad", [(5000, None), (4099, 8)])
def test_small_multitile(gpu, tdt, ddt, V, pad, grouping):
    H.log(f"early exit small multitile tdt={tdt} ddt={ddt} V={V} pad={pad}")
    inp = synth.make_custom_sample(6, 3, V, tdt, ddt, T=[0.5, 0.9, 1.0, 1.3, 2.0, 0.7], noise_sd=0.8, seed=V + 1)
    _both(gpu, inp, pad=pad, name=f"{tdt}/{ddt} V={V}", grouping=grouping)


def test_config1_tiny(gpu):
    H.log("early exit config 1: 10^4 trials, gamma=4, V=32, shared logits")
    _both(gpu, synth.make_sample_inputs(1, seed=0), name="config1")


def test_config2(gpu):
    H.log("early exit config 2: B=64 gamma=4 V=32000 bf16")
    _both(gpu, synth.make_sample_inputs(2, seed=0), name="config2")


def test_config3(gpu):
    H.log("early exit config 3: B=256 gamma=8 V=128256 bf16 (all vs one pass, 32 vs oracle)")
    inp = synth.make_sample_inputs(3, seed=0)
    seqs = sorted(set(np.random.default_rng(33).choice(inp.B, 30, replace=False).tolist()) | {0, inp.B - 1})
    ee = _both(gpu, inp, seqs=seqs, name="config3")
    assert (ee["n"] >= 0).all()


def test_config5(gpu):
    H.log("early exit config 5: B=512 gamma=5 V=256000 bf16/fp32 (all vs one pass, 24 vs oracle)")
    inp = synth.make_sample_inputs(5, seed=0)
    rng = np.random.default_rng(55)
    seqs = []
    for cls in (0, 1, 2):
        seqs += rng.choice(np.flatnonzero(inp.row_class == cls), 8, replace=False).tolist()
    ee = _both(gpu, inp, seqs=sorted(seqs), name="config5")
    assert (ee["n"][inp.row_class == 2] == inp.gamma).all()


@pytest.mark.parametrize("grouping", GROUPINGS)
@pytest.mark.parametrize("G", [1, 16, 64])
def test_gamma_extremes(gpu, G, grouping):
    H.log(f"early exit gamma={G}")
    inp = synth.make_custom_sample(5, G, 3000, "bf16", "f32", T=1.0, noise_sd=0.3, seed=G + 100)
    _both(gpu, inp, name=f"gamma {G}", grouping=grouping)


@pytest.mark.parametrize("grouping", GROUPINGS)
@pytest.mark.parametrize("case", ["masks_and_signed_zero", "identical_and_disjoint", "invalid_inputs",
                                  "unconsulted_positions", "invalid_after_accepts"])
def test_edge_cases(gpu, case, grouping):
    H.log(f"early exit edge case {case} ({grouping})")
    inp = getattr(SC, case)()
    ee = _both(gpu, inp, name=case, grouping=grouping)
    if case == "invalid_inputs":
        assert (ee["n"] == -1).all()
    if case == "invalid_after_accepts":
        assert list(ee["n"]) == [-1, -1, -1, 1]


def test_garbage_workspace_and_alternation(gpu):
    """The workspace needs no initialisation, and the two entry points can
    share one workspace in any order."""
    H.log("early exit garbage workspace")
    ws = gpu.Workspace()
    ws.buf = torch.randint(0, 255, (64 << 20,), dtype=torch.uint8, device="cuda")
    a = SC.custom(9, 6, 5000, "bf16", "bf16", seed=21)
    b = SC.custom(3, 2, 800, "f32", "bf16", seed=22)
    ta, tb = H.sample_tensors(a), H.sample_tensors(b)
    ref_a = H.run_sample(gpu, ta, early_exit=True)
    for early in (True, False, True):
        H.run_sample(gpu, tb, workspace=ws, early_exit=not early)
        r = H.run_sample(gpu, ta, workspace=ws, early_exit=early)
        assert np.array_equal(r["n"], ref_a["n"]) and np.array_equal(r["tokens"], ref_a["tokens"])
    assert not H.check_sample(a, ref_a).fail


def test_repeat_calls_bit_identical(gpu):
    inp = SC.custom(16, 5, 20000, "bf16", "f32", seed=23)
    tens = H.sample_tensors(inp)
    r1 = H.run_sample(gpu, tens, early_exit=True)
    r2 = H.run_sample(gpu, tens, early_exit=True)
    for k in r1:
        assert np.array_equal(r1[k].view(np.uint8), r2[k].view(np.uint8)), k


@pytest.mark.parametrize("grouping", GROUPINGS)
@pytest.mark.parametrize("T", [1e-6, 1e-12, 1e-30])
def test_temperature_extremes(gpu, T, grouping):
    H.log(f"early exit T={T}")
    inp = synth.make_custom_sample(6, 4, 2048, "bf16", "f32", T=T, noise_sd=0.5, seed=12)
    _both(gpu, inp, name=f"T={T}", grouping=grouping)


@pytest.mark.parametrize("grouping", GROUPINGS)
def test_huge_logits(gpu, grouping):
    """Logits around 10^8 (N(0, 2e7)): the statistics pass takes its subtract form."""
    inp = synth.make_custom_sample(6, 3, 3000, "f32", "f32", T=1.0, noise_sd=1e6, target_sd=2e7, seed=13)
    _both(gpu, inp, name="huge logits", grouping=grouping)


@pytest.mark.parametrize("tdt,ddt", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("V", [32, 700, 2048, 5000, 40000])
def test_one_step_rows_no_gate_same_bits(gpu, tdt, ddt, V):
    """No gated position (a small call: the grouping chosen from the sizes, or
    tail_start = 0): the early exit reads every row in any case and runs the
    one-pass call (its one-kernel path for V <= 2048), so its outputs and
    diagnostics equal the one-pass call's bit for bit, and match the oracle."""
    H.log(f"early exit, no gate: V={V} {tdt}/{ddt}")
    inp = synth.make_custom_sample(40, 4, V, tdt, ddt, T=np.linspace(0.5, 1.5, 40, dtype=np.float32),
                                   noise_sd=0.6, seed=V + 7)
    tens = H.sample_tensors(inp, pad_to=8)  # rows padded to 16 bytes (V = 700 in bf16)
    one = H.run_sample(gpu, tens)
    for ts in (None, 0):
        ee = H.run_sample(gpu, tens, early_exit=True, tail_start=ts)
        for k in one:
            assert np.array_equal(one[k].view(np.uint8), ee[k].view(np.uint8)), (k, ts)
    t = H.check_sample(inp, one)
    H.log(f"[early exit one-step rows V={V}] {t.summary()}")
    assert not t.fail, t.fail[:3]


@pytest.mark.parametrize("grouping", ["first", "all"])
@pytest.mark.parametrize("V,tdt,ddt", [(32, "f32", "f32"), (20, "bf16", "bf16"), (700, "bf16", "f32")])
def test_one_step_rows_gated(gpu, V, tdt, ddt, grouping):
    """Rows of one draw step with gated positions: the statistics launches and
    the finish kernel (not the one-kernel path), against the oracle and the
    one-pass call."""
    H.log(f"early exit, rows of one step, gated ({grouping}): V={V} {tdt}/{ddt}")
    inp = synth.make_custom_sample(9, 5, V, tdt, ddt, T=np.linspace(0.6, 1.4, 9, dtype=np.float32),
                                   noise_sd=0.6, seed=V + 17)
    _both(gpu, inp, pad=8, name=f"one-step rows V={V}", grouping=grouping)
