"""GPU edge cases against the oracle: ragged and tiny vocabularies, extreme
gamma and temperature, masks, signed zeros, invalid inputs, strided rows,
workspace reuse across shapes, the staged entry point, and tree corner cases."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec_verify_oracle as O
from tests import gpu_helpers as H
from tests import sample_cases as SC

pytestmark = pytest.mark.gpu


def _check(inp, out, name, allow_flags=2):
    t = H.check_sample(inp, out)
    H.log(f"[{name}] {t.summary()}")
    assert not t.fail, t.fail[:5]
    assert t.flagged <= allow_flags
    return t


@pytest.mark.parametrize("V", [1, 7, 8, 9, 31, 33, 2047, 2048, 2049, 4097, 128257])
@pytest.mark.parametrize("tdt,ddt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_vocab_sizes(gpu, V, tdt, ddt):
    """Up to 2048 tokens the full call runs the one-wave-per-sequence kernel;
    the staged (two-kernel) path is checked at every size too."""
    H.log(f"vocab V={V} {tdt}/{ddt}")
    inp = synth.make_custom_sample(5, 3, V, tdt, ddt, T=[0.6, 1.0, 1.0, 1.5, 0.9], seed=V + 1)
    tens = H.sample_tensors(inp, pad_to=8)
    out = H.run_sample(gpu, tens)
    _check(inp, out, f"V={V}")
    if V == 1:
        assert (out["n"] == 3).all() and (out["tokens"] == 0).all()
    _check(inp, H.run_sample_staged(gpu, tens), f"V={V} staged")


@pytest.mark.parametrize("V", [3000, 696])
@pytest.mark.parametrize("G", [1, 16, 64])
def test_gamma_extremes(gpu, G, V):
    H.log(f"gamma={G} V={V}")
    inp = synth.make_custom_sample(4, G, V, "bf16", "bf16", T=1.0, noise_sd=0.3, seed=G)
    _full_and_staged(gpu, inp, f"gamma={G} V={V}")


@pytest.mark.parametrize("T", [0.05, 10.0, 1e-6, 1e-12, 1e-30])
def test_temperature_extremes(gpu, T):
    H.log(f"T={T}")
    inp = synth.make_custom_sample(6, 4, 2048, "bf16", "f32", T=T, noise_sd=0.5, seed=11)
    _full_and_staged(gpu, inp, f"T={T}")


def test_vocab_beyond_lds_steps(gpu):
    """V = 4.2M: the draw's step masses (2051 steps) live in the workspace, not LDS."""
    inp = synth.make_custom_sample(2, 1, 4_200_000, "f32", "f32", T=1.0, noise_sd=0.5, seed=14)
    _check(inp, H.run_sample(gpu, H.sample_tensors(inp)), "V=4.2M")


def test_batch_of_one(gpu):
    inp = synth.make_custom_sample(1, 5, 50000, "f32", "bf16", T=0.8, seed=3)
    _check(inp, H.run_sample(gpu, H.sample_tensors(inp)), "B=1")


_custom = SC.custom


def _full_and_staged(gpu, inp, name):
    """The full call and the two kernels one stage at a time, both against the
    oracle (at up to 2048 tokens the full call is the one-wave kernel); returns
    both results."""
    tens = H.sample_tensors(inp)
    out = H.run_sample(gpu, tens)
    _check(inp, out, name)
    staged = H.run_sample_staged(gpu, tens)
    _check(inp, staged, name + " staged")
    return out, staged


def test_masks_and_signed_zero(gpu):
    _full_and_staged(gpu, SC.masks_and_signed_zero(), "masks")


def test_identical_and_disjoint_rows(gpu):
    for out in _full_and_staged(gpu, SC.identical_and_disjoint(), "identical/disjoint"):
        assert (out["n"][:4] == 5).all() and (out["n"][4:] == 0).all()
        assert (out["tokens"][4:, 0] < 1500).all()


def test_invalid_inputs(gpu):
    for out in _full_and_staged(gpu, SC.invalid_inputs(), "invalid"):
        assert (out["n"] == -1).all() and (out["tokens"] == -1).all()


def test_unconsulted_positions_are_ignored(gpu):
    """Rows, tokens and uniforms after the first rejection do not matter."""
    for out in _full_and_staged(gpu, SC.unconsulted_positions(), "unconsulted"):
        assert (out["n"] == 0).all()


def test_invalid_after_accepts(gpu):
    for out in _full_and_staged(gpu, SC.invalid_after_accepts(), "invalid after accepts"):
        assert list(out["n"]) == [-1, -1, -1, 1]


def test_strided_rows(gpu):
    inp = synth.make_custom_sample(6, 3, 3000, "bf16", "f32", T=0.9, seed=8)
    tens = H.sample_tensors(inp)
    # embed in wider rows and a batch with gaps: row stride 3064, sequence stride 2 * 4 rows
    t_big = torch.full((12, 4, 3064), float("nan"), dtype=torch.bfloat16, device="cuda")
    d_big = torch.full((12, 3, 3064), float("nan"), dtype=torch.float32, device="cuda")
    t_big[::2, :, :3000] = tens["target"]
    d_big[::2, :, :3000] = tens["draft"]
    tens["target"] = t_big[::2, :, :3000]
    tens["draft"] = d_big[::2, :, :3000]
    assert tens["target"].stride() == (2 * 4 * 3064, 3064, 1)
    _check(inp, H.run_sample(gpu, tens), "strided")


def test_workspace_reuse_across_shapes_and_stages(gpu):
    """A garbage-filled workspace reused across shapes gives the same results."""
    ws = gpu.Workspace()
    ws.buf = torch.randint(0, 255, (64 << 20,), dtype=torch.uint8, device="cuda")  # no initialisation needed
    a = _custom(5, 3, 4000, "bf16", "bf16", seed=9)
    b = _custom(17, 6, 1000, "f32", "bf16", seed=10)
    ta, tb = H.sample_tensors(a), H.sample_tensors(b)
    ra1 = H.run_sample(gpu, ta, workspace=ws)
    rb = H.run_sample(gpu, tb, workspace=ws)
    ra2 = H.run_sample(gpu, ta, workspace=ws)
    _check(a, ra1, "ws a")
    _check(b, rb, "ws b")
    for k in ra1:
        assert np.array_equal(ra1[k], ra2[k], equal_nan=True)
    # staged entry point: stages 1, 2 equal the full call
    n = torch.empty(5, dtype=torch.int32, device="cuda")
    t = torch.empty((5, 4), dtype=torch.int32, device="cuda")
    for stage in (1, 2):
        gpu.spec_verify_sample_stage(stage, **ta, out_num_accepted=n, out_tokens=t, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(n.cpu().numpy(), ra1["n"]) and np.array_equal(t.cpu().numpy(), ra1["tokens"])
    # no diagnostics requested
    r = H.run_sample(gpu, ta, diag=False, workspace=ws)
    assert np.array_equal(r["n"], ra1["n"])


@pytest.mark.parametrize("B,G,V,tdt,ddt", [(24, 3, 70000, "bf16", "f32"), (3, 2, 300000, "f32", "bf16"),
                                         (40, 2, 128256, "bf16", "bf16"), (1, 4, 256000, "bf16", "f32"),
                                         (128, 2, 70000, "bf16", "bf16"), (100, 2, 100000, "bf16", "f32")])
def test_finish_split_over_parts(gpu, B, G, V, tdt, ddt):
    """Few sequences with long rows: each sequence's draw is split over several
    finish workgroups (the last to finish gathers the step masses and draws):
    16-wave parts where the parts' streams are short (the first four shapes),
    8-wave parts where they are long (B = 128 and 100: 2 and 3 parts).
    Results against the oracle; then the finish stage alone, run three times
    after one statistics stage on a garbage-filled workspace, gives the full
    call's outputs every time (the hand-off state is reset by the statistics
    pass and again by the drawing part)."""
    H.log(f"finish parts B={B} G={G} V={V} {tdt}/{ddt}")
    inp = synth.make_custom_sample(B, G, V, tdt, ddt, T=0.8, noise_sd=0.6, seed=B + V)
    tens = H.sample_tensors(inp)
    ws = gpu.Workspace()
    ws.buf = torch.randint(0, 255, (gpu.sv_sample_workspace_bytes(B, G, V) + 4096,), dtype=torch.uint8,
                           device="cuda")
    full = H.run_sample(gpu, tens, workspace=ws)
    _check(inp, full, f"parts B={B} V={V}")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    t = torch.empty((B, G + 1), dtype=torch.int32, device="cuda")
    ws.buf.random_(0, 255)
    gpu.spec_verify_sample_stage(1, **tens, out_num_accepted=n, out_tokens=t, workspace=ws)
    for rep in range(3):
        n.fill_(-7)
        t.fill_(-7)
        gpu.spec_verify_sample_stage(2, **tens, out_num_accepted=n, out_tokens=t, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(n.cpu().numpy(), full["n"]), rep
        assert np.array_equal(t.cpu().numpy(), full["tokens"]), rep
    ee = H.run_sample(gpu, tens, workspace=ws, early_exit=True)
    differ, bad = H.compare_one_pass(full, ee)
    assert not bad, bad[:5]
    _check(inp, ee, f"parts early exit B={B} V={V}")


def test_bad_arguments_raise(gpu):
    inp = _custom(2, 2, 64, "f32", "f32")
    tens = H.sample_tensors(inp)
    with pytest.raises(ValueError):
        gpu.spec_verify_sample(tens["target"].to(torch.float16), tens["draft"], tens["draft_tokens"],
                               tens["uniforms"], tens["temperature"])
    bad = dict(tens)
    bad["target"] = torch.zeros((2, 3, 70), dtype=torch.bfloat16, device="cuda")[:, :, 1:65]  # misaligned rows
    with pytest.raises(ValueError):
        gpu.spec_verify_sample(**bad)


# ---------------------------------------------------------------------------
# tree
# ---------------------------------------------------------------------------
def _tree_run_check(gpu, logits, parents, tokens, dt="f32"):
    tens = dict(logits=H.dev_logits(logits, dt), parents=torch.from_numpy(parents).cuda(),
                tokens=torch.from_numpy(tokens).cuda())
    out = H.run_tree(gpu, tens)
    fails = H.check_tree(logits, dt, parents, tokens, out)
    assert not fails, fails[:3]
    return out


def test_tree_golden_cases(gpu):
    from tests.golden_io import farray, load

    for case in load("tree_cases.json"):
        L = farray(case["logits"]).astype(np.float32)
        V = L.shape[1]
        Lp = np.zeros((L.shape[0], 4), np.float32)  # rows padded to 16 bytes
        Lp[:, :V] = L
        tens = dict(logits=H.dev_logits(Lp[None], "f32")[..., :V],
                    parents=torch.tensor([case["parents"]], dtype=torch.int32, device="cuda"),
                    tokens=torch.tensor([case["tokens"]], dtype=torch.int32, device="cuda"))
        out = H.run_tree(gpu, tens)
        if case["valid"]:
            assert int(out["len"][0]) == case["accept_len"], case["name"]
            assert list(out["path"][0][: len(case["path"])]) == case["path"], case["name"]
            assert int(out["bonus"][0]) == case["bonus"], case["name"]
            assert list(out["argmax"][0]) == case["argmax"], case["name"]
        else:
            assert int(out["len"][0]) == -1 and int(out["bonus"][0]) == -1, case["name"]


def test_tree_ties_zero_masks(gpu):
    g = np.random.default_rng(12)
    B, N, V = 16, 40, 4099
    parents = np.array([[-1] + [int(g.integers(0, j)) for j in range(1, N)] for _ in range(B)], np.int32)
    L = g.integers(-3, 4, size=(B, N, V)).astype(np.float32)  # many exact ties
    L[g.random(L.shape) < 0.1] = -0.0
    L[g.random(L.shape) < 0.2] = -np.inf
    L[3, 5, :] = -np.inf  # a row of -inf only
    tokens = g.integers(0, 4, size=(B, N)).astype(np.int32)  # low tokens: many matches, duplicate siblings
    for dt in ("f32", "bf16"):
        Ld = L if dt == "f32" else synth.f32_to_bf16_bits(L)
        Lp = np.full((B, N, 4104), np.nan, np.float32) if dt == "f32" else np.full((B, N, 4104), 0x7FC1, np.uint16)
        Lp[..., :V] = Ld
        tens = dict(logits=H.dev_logits(Lp, dt)[..., :V], parents=torch.from_numpy(parents).cuda(),
                    tokens=torch.from_numpy(tokens).cuda())
        out = H.run_tree(gpu, tens)
        fails = H.check_tree(Ld, dt, parents, tokens, out)
        assert not fails, fails[:3]


def test_tree_invalid(gpu):
    g = np.random.default_rng(13)
    B, N, V = 6, 9, 256
    L = g.normal(size=(B, N, V)).astype(np.float32)
    parents = np.array([[-1] + list(range(N - 1))] * B, np.int32)
    tokens = g.integers(0, V, size=(B, N)).astype(np.int32)
    L[0, 3, 7] = np.nan
    L[1, 8, 0] = np.inf
    parents[2, 4] = 4
    parents[3, 0] = 0
    tokens[4, 2] = V
    out = _tree_run_check(gpu, L, parents, tokens)
    assert (out["len"][:5] == -1).all() and out["len"][5] >= 0
    assert out["argmax"][0, 3] == -1 and out["argmax"][1, 8] == -1


@pytest.mark.parametrize("N", [63, 64, 65])
def test_tree_one_wave_boundary(gpu, N):
    """Trees of up to 64 nodes resolve in one wave (registers), larger ones in
    LDS: at N = 63, 64 and 65, a full chain whose edges all match, the same
    chain broken half way, a star, random trees with repeated sibling tokens
    (ties on depth go to the lowest id), and an invalid tree in the batch, all
    bit-exact against the oracle."""
    g = np.random.default_rng(300 + N)
    V = 40
    B = 7
    L = g.integers(-3, 4, size=(B, N, V)).astype(np.float32)  # many exact ties
    parents = np.empty((B, N), np.int32)
    parents[0] = parents[1] = [-1] + list(range(N - 1))
    parents[2] = [-1] + [0] * (N - 1)
    for b in range(3, B):
        parents[b] = [-1] + [int(g.integers(max(0, j - 4), j)) for j in range(1, N)]
    am = np.argmax(L, axis=2)  # lowest index on ties
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for j in range(1, N):
            p = parents[b, j]
            tokens[b, j] = am[b, p] if (b < 2 or g.random() < 0.7) else (am[b, p] + 1) % V
    tokens[1, N // 2] = (am[1, N // 2 - 1] + 1) % V  # the second chain breaks at node N / 2
    parents[6, 5] = 9  # a forward parent: invalid tree
    out = _tree_run_check(gpu, L, parents, tokens)
    assert out["len"][0] == N - 1 and out["len"][1] == N // 2 - 1
    assert out["len"][2] == 1 and out["len"][6] == -1 and (out["path"][6] == -1).all()


def test_tree_single_node_and_max_chain(gpu):
    g = np.random.default_rng(14)
    L = g.normal(size=(3, 1, 64)).astype(np.float32)
    out = _tree_run_check(gpu, L, np.full((3, 1), -1, np.int32), np.zeros((3, 1), np.int32))
    assert (out["len"] == 0).all()
    N, V = 1024, 64
    L = g.normal(size=(2, N, V)).astype(np.float32)
    parents = np.array([[-1] + list(range(N - 1))] * 2, np.int32)
    tokens = np.zeros((2, N), np.int32)
    for j in range(1, N):
        tokens[:, j] = np.argmax(L[:, j - 1], axis=1)  # every edge matches
    tokens[1, 700] = (tokens[1, 700] + 1) % V  # second chain breaks at node 700
    out = _tree_run_check(gpu, L, parents, tokens)
    assert out["len"][0] == N - 1 and out["len"][1] == 699


@pytest.mark.parametrize("V", [1, 7, 33])
def test_tree_tiny_vocab(gpu, V):
    ti = synth.make_tree_inputs(4, seed=V, B=5, N=30, V=max(V, 8), dtype="f32")
    L = ti.logits[..., :V].copy()
    Lp = np.full(ti.logits.shape[:2] + (8 * ((V + 7) // 8),), np.nan, np.float32)
    Lp[..., :V] = L
    tokens = np.minimum(ti.tokens, V - 1).astype(np.int32)
    tens = dict(logits=H.dev_logits(Lp, "f32")[..., :V], parents=torch.from_numpy(ti.parents).cuda(),
                tokens=torch.from_numpy(tokens).cuda())
    out = H.run_tree(gpu, tens)
    fails = H.check_tree(L, "f32", ti.parents, tokens, out)
    assert not fails, fails[:3]


def test_tree_stages_equal_full_call(gpu):
    ti = synth.make_tree_inputs(4, seed=15, B=4, N=20, V=5000)
    tens = H.tree_tensors(ti)
    full = H.run_tree(gpu, tens)
    ws = gpu.Workspace()
    ws.buf = torch.randint(0, 255, (8 << 20,), dtype=torch.uint8, device="cuda")
    outs = None
    for stage in (1, 2):
        outs = gpu.spec_verify_greedy_tree_stage(stage, **tens, workspace=ws) if outs is None else \
            gpu.spec_verify_greedy_tree_stage(stage, **tens, out_accept_len=outs[0], out_path=outs[1],
                                              out_bonus=outs[2], out_argmax=outs[3], workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(outs[0].cpu().numpy(), full["len"])
    assert np.array_equal(outs[1].cpu().numpy(), full["path"])
    assert np.array_equal(outs[2].cpu().numpy(), full["bonus"])
    assert np.array_equal(outs[3].cpu().numpy(), full["argmax"])


def test_prepared_calls_repeat_the_direct_calls(gpu):
    """Calls prepared once (prepare=True) enqueue the same work each time they
    are called: their outputs equal the direct calls' on every repetition."""
    inp = _custom(9, 4, 20000, "bf16", "f32", seed=21)
    tens = H.sample_tensors(inp)
    ws = gpu.Workspace()
    direct = H.run_sample(gpu, tens, diag=False, workspace=ws)
    call = gpu.spec_verify_sample(**tens, workspace=ws, prepare=True)
    ee = gpu.spec_verify_sample_early_exit(**tens, workspace=ws, prepare=True)
    for rep in range(3):
        for c in (call, ee):
            c.outputs[0].fill_(-7)
            n, t, _ = c()
            torch.cuda.synchronize()
            assert np.array_equal(n.cpu().numpy(), direct["n"]), rep
            assert np.array_equal(t.cpu().numpy(), direct["tokens"]), rep

    ti = synth.make_tree_inputs(4, seed=16, B=3, N=25, V=3000)
    tt = H.tree_tensors(ti)
    full = H.run_tree(gpu, tt)
    tcall = gpu.spec_verify_greedy_tree(**tt, prepare=True)
    for rep in range(2):
        tcall.outputs[0].fill_(-7)
        out = tcall()
        torch.cuda.synchronize()
        assert np.array_equal(out[0].cpu().numpy(), full["len"]) and np.array_equal(out[2].cpu().numpy(),
                                                                                      full["bonus"]), rep

    d = synth.make_draft_rows(6, 5000, "bf16", T=0.9, seed=22)
    dt = H.draft_tensors(d)
    y0, p0 = gpu.spec_draft_sample(**dt, want_prob=True)
    dcall = gpu.spec_draft_sample(**dt, want_prob=True, prepare=True)
    for rep in range(2):
        dcall.outputs[0].fill_(-7)
        y, p = dcall()
        torch.cuda.synchronize()
        assert torch.equal(y, y0) and torch.equal(p, p0), rep

    par = torch.from_numpy(ti.parents).cuda()
    m0, _, d0 = gpu.spec_tree_mask(par)
    mcall = gpu.spec_tree_mask(par, prepare=True)
    mcall.outputs[0].fill_(7)
    m, _, dd = mcall()
    torch.cuda.synchronize()
    assert torch.equal(m, m0) and torch.equal(dd, d0)


def test_split_finish_repeats_bit_identical(gpu):
    """A split finish (16 sequences of 200k tokens: 12 parts each) gives the
    same bits on every call, diagnostics included, whichever step masses the
    drawing part found published and whichever it recomputed."""
    inp = synth.make_custom_sample(16, 3, 200000, "bf16", "f32", T=0.9, noise_sd=0.7, seed=31)
    tens = H.sample_tensors(inp)
    first = H.run_sample(gpu, tens)
    _check(inp, first, "split repeat")
    for rep in range(4):
        again = H.run_sample(gpu, tens)
        for k in first:
            assert np.array_equal(first[k].view(np.uint8), again[k].view(np.uint8)), (rep, k)


@pytest.mark.parametrize("G", [31, 32, 63, 64])
def test_full_acceptance_at_large_gamma(gpu, G):
    """Draft rows equal to the target rows: every draft is accepted and the
    token comes from the bonus row gamma, whose statistics are the last of the
    2 gamma + 1 rows (more rows than lanes in the one-wave kernel)."""
    inp = synth.make_custom_sample(4, G, 696, "bf16", "bf16", T=0.9, noise_sd=0.0, seed=40 + G)
    for out in _full_and_staged(gpu, inp, f"full acceptance gamma={G}"):
        assert (out["n"] == G).all()


@pytest.mark.parametrize("tdt,ddt,T", [("bf16", "f32", 1e-7), ("f32", "bf16", 1e-7), ("bf16", "bf16", 1.0)])
def test_one_step_per_wave_finish(gpu, tdt, ddt, T):
    """One finish workgroup per sequence with at most one step per wave (V =
    5000, 3 steps): the waves keep their steps and the drawing wave rescans
    from registers, in the FMA form and (T = 1e-7: shifts beyond 2^24) the
    subtract form; against the oracle, and the staged kernels give the same
    bits."""
    H.log(f"one step per wave: {tdt}/{ddt} T={T}")
    inp = synth.make_custom_sample(6, 3, 5000, tdt, ddt, T=T, noise_sd=0.5, seed=61)
    out, staged = _full_and_staged(gpu, inp, f"one step per wave {tdt}/{ddt} T={T}")
    for k in out:
        assert np.array_equal(out[k].view(np.uint8), staged[k].view(np.uint8)), k


@pytest.mark.parametrize("V,tdt,ddt", [(5000, "bf16", "f32"), (128257, "bf16", "bf16"), (1500, "f32", "f32")])
def test_read_stage_writes_no_output(gpu, V, tdt, ddt):
    """Stage 3 (the statistics pass's reads alone, a measurement) leaves every
    output as it was, and the full call on the same workspace afterwards still
    gives the oracle's results (the statistics pass resets what stage 3 may
    have left in the workspace)."""
    H.log(f"read stage V={V} {tdt}/{ddt}")
    inp = synth.make_custom_sample(6, 4, V, tdt, ddt, T=[0.7, 1.0, 1.3, 0.9, 1.0, 2.0], seed=V + 7)
    tens = H.sample_tensors(inp, pad_to=8)
    ws = gpu.Workspace()
    B, G = inp.tokens.shape
    n0 = torch.full((B,), -77, dtype=torch.int32, device="cuda")
    t0 = torch.full((B, G + 1), -77, dtype=torch.int32, device="cuda")
    gpu.spec_verify_sample_stage(3, **tens, out_num_accepted=n0, out_tokens=t0, workspace=ws)
    torch.cuda.synchronize()
    assert (n0.cpu().numpy() == -77).all() and (t0.cpu().numpy() == -77).all()
    _check(inp, H.run_sample_staged(gpu, tens, workspace=ws), f"after read stage V={V}")
