"""Checks of the seeded input generators (CPU)."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec_verify_oracle as O


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    vals = np.concatenate([
        g.normal(0, 3, 20000).astype(np.float32),
        np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 3.3895314e38, 3.4e38, 1e-40, -0.0,
                  np.inf, -np.inf], dtype=np.float32),
    ])
    mine = synth.f32_to_bf16_bits(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    assert synth.f32_to_bf16_bits(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80  # tie -> even
    assert synth.f32_to_bf16_bits(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 0x3F82
    nan = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    back = synth.bf16_bits_to_f32(mine[:20000])
    np.testing.assert_array_equal(back, torch.from_numpy(mine[:20000].view(np.int16)).view(torch.bfloat16).float().numpy())


def test_uniforms_are_exact_u24():
    u = synth.uniforms_u24(synth.gen(0, 9, 4), (1000, 7))
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()
    k = u.astype(np.float64) * 2 ** 24
    assert np.array_equal(k, np.floor(k))


def test_determinism_per_sequence():
    a = synth.make_sample_inputs(3, seed=5, B=3)
    b = synth.make_sample_inputs(3, seed=5, B=3)
    for f in ("target", "draft", "tokens", "uniforms", "temperature"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


@pytest.mark.parametrize("cid", [2, 3])
def test_alpha_near_goal(cid):
    inp = synth.make_sample_inputs(cid, seed=0, B=4)
    cfg = synth.CONFIGS[cid]
    al = []
    for b in range(inp.B):
        T = float(inp.temperature[b])
        for i in range(inp.gamma):
            p = O.tempered_softmax(O.widen(inp.target[b, i], cfg.target_dtype), T)[0]
            q = O.tempered_softmax(O.widen(inp.draft[b, i], cfg.draft_dtype), T)[0]
            al.append(O.alpha(p, q))
    assert abs(np.mean(al) - cfg.alpha_goal) < 0.03, np.mean(al)


def test_config5_normal_rows_alpha_near_goal():
    """Configuration 5's normal rows: mean alpha within 0.03 of the goal 0.7
    over 12 sequences (60 positions) of the workload's own rows (seed 0, B =
    512), each at its per-row temperature."""
    cfg = synth.CONFIGS[5]
    cls = synth.row_classes(cfg, 0)
    temps = synth.temperatures(cfg, 0, cfg.B)
    scale = synth.draft_noise_scale(5)
    al = []
    for b in np.flatnonzero(cls == 0)[:12]:
        t32 = synth.target_rows(cfg, 0, int(b), cfg.gamma + 1)
        tr = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(t32))
        d = synth.draft_rows(cfg, 0, int(b), tr, scale, 0, float(temps[b]))
        T = float(temps[b])
        for i in range(cfg.gamma):
            al.append(O.alpha(O.tempered_softmax(tr[i].astype(np.float64), T)[0],
                              O.tempered_softmax(d[i].astype(np.float64), T)[0]))
    assert abs(np.mean(al) - cfg.alpha_goal) < 0.03, np.mean(al)


def test_config5_row_classes():
    cfg = synth.CONFIGS[5]
    cls = synth.row_classes(cfg, 0)
    assert (cls == 1).sum() == 51 and (cls == 2).sum() == 51 and (cls == 0).sum() == 410
    temps = synth.temperatures(cfg, 0, cfg.B)
    assert temps.min() >= 0.3 and temps.max() <= 1.5
    # a few sequences of each class, built exactly as make_sample_inputs does
    idx = {c: int(np.flatnonzero(cls == c)[0]) for c in (0, 1, 2)}
    scale = synth.draft_noise_scale(5)
    for c, b in idx.items():
        t32 = synth.target_rows(cfg, 0, b, cfg.gamma + 1)
        tq = synth.f32_to_bf16_bits(t32)
        tr = synth.bf16_bits_to_f32(tq)
        d = synth.draft_rows(cfg, 0, b, tr, scale, c, float(temps[b]))
        T = float(temps[b])
        al = [O.alpha(O.tempered_softmax(tr[i].astype(np.float64), T)[0],
                      O.tempered_softmax(d[i].astype(np.float64), T)[0]) for i in range(cfg.gamma)]
        if c == 2:
            assert np.array_equal(d, tr[: cfg.gamma])
            assert min(al) > 1 - 1e-12
        elif c == 1:
            assert max(al) < 1e-3
            assert np.isfinite(d).sum(axis=1).min() > 1000
        else:
            assert 0.4 < np.mean(al) < 0.95


def test_draft_tokens_never_masked():
    inp = synth.make_sample_inputs(5, seed=0, B=24)
    for b in range(inp.B):
        for i in range(inp.gamma):
            assert np.isfinite(inp.draft[b, i, inp.tokens[b, i]])


def test_tree_shape_constraints():
    ti = synth.make_tree_inputs(4, seed=0)
    cfg = synth.CONFIGS[4]
    assert ti.parents.shape == (32, 60)
    for b in range(ti.parents.shape[0]):
        par = ti.parents[b]
        assert par[0] == -1 and all(0 <= par[j] < j for j in range(1, 60))
        depth = np.zeros(60, int)
        for j in range(1, 60):
            depth[j] = depth[par[j]] + 1
        assert depth.max() <= cfg.max_depth
        kids = {}
        for j in range(1, 60):
            kids.setdefault(int(par[j]), []).append(j)
        for p, ks in kids.items():
            toks = [int(ti.tokens[b, k]) for k in ks]
            assert len(set(toks)) == len(toks)  # distinct sibling tokens
            if depth[p] % 2 == 1:
                assert len(ks) == 1  # inside a 2-token block: a chain
            elif max(ks) < 59 and depth[p] < 4:
                assert 2 <= len(ks) <= 4
    # about 75% of edges planted
    frac = ti.planted.sum() / max(1, sum(len(set(ti.parents[b][1:])) for b in range(32)))
    assert 0.6 < frac < 0.9
