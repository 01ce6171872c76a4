"""Host-side checks of the benchmark (no GPU): the byte counts the roofline
divides by, counted here independently element by element from the shapes of
the tensors each kernel touches, and the refusal of more than one GPU."""
import subprocess
import sys
import types

import numpy as np

import bench


def _cfg(tdt, ddt):
    return types.SimpleNamespace(target_dtype=tdt, draft_dtype=ddt)


def test_sample_bytes_counted_per_tensor():
    """Stats: every target row (gamma + 1 per sequence) and draft row (gamma)
    once, plus the int32 tokens, fp32 uniforms (gamma + 1) and temperature.
    Finish: per sequence, the target row at its stop position and, after a
    rejection, the draft row there too, plus its int32 outputs (count and
    gamma + 1 tokens)."""
    B, G, V = 7, 5, 1000
    n_acc = np.array([0, 5, 2, 5, 4, -1, 1])  # -1: an invalid sequence counts as a rejection
    for tdt, ddt, bt, bd in (("bf16", "f32", 2, 4), ("bf16", "bf16", 2, 2), ("f32", "f32", 4, 4)):
        target = np.zeros((B, G + 1, V), dtype=np.uint8 if bt == 1 else (np.uint16 if bt == 2 else np.uint32))
        draft = np.zeros((B, G, V), dtype=np.uint16 if bd == 2 else np.uint32)
        tokens = np.zeros((B, G), dtype=np.int32)
        uniforms = np.zeros((B, G + 1), dtype=np.float32)
        temps = np.zeros(B, dtype=np.float32)
        s1_want = target.nbytes + draft.nbytes + tokens.nbytes + uniforms.nbytes + temps.nbytes
        s2_want = 0
        for b in range(B):
            s2_want += V * bt  # the target row the draw reads
            if n_acc[b] < G:
                s2_want += V * bd  # and the draft row beside it after a rejection
            s2_want += 4 + (G + 1) * 4  # n and the token list
        s1, s2 = bench.sample_bytes(_cfg(tdt, ddt), B, G, V, n_acc)
        assert s1 == s1_want, (tdt, ddt, s1, s1_want)
        assert s2 == s2_want, (tdt, ddt, s2, s2_want)


def test_c5_stats_bytes():
    """The headline call: 512 sequences of 6 bf16 target rows and 5 fp32 draft
    rows of 256000 logits are 4 194 304 000 bytes of logits."""
    s1, _ = bench.sample_bytes(_cfg("bf16", "f32"), 512, 5, 256000)
    logits = 512 * 6 * 256000 * 2 + 512 * 5 * 256000 * 4
    assert logits == 4_194_304_000
    assert s1 == logits + 512 * (5 * 4 + 6 * 4 + 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120,
                       cwd=bench.__file__.rsplit("/", 1)[0])
    assert r.returncode == 2
    assert "exactly one GPU" in r.stdout


def test_early_exit_bytes_counted_per_row():
    """Early exit reads, per sequence stopped at position n, the target rows
    0..n and the draft rows 0..n (0..gamma-1 after full acceptance; every row
    of an invalid sequence), then the finish's bytes as in the one-pass call,
    plus the per-position inputs."""
    B, G, V = 6, 4, 300
    n_acc = np.array([0, 4, 2, -1, 3, 1])
    cfg = _cfg("bf16", "f32")
    want = 0
    for b in range(B):
        n = G if n_acc[b] < 0 else n_acc[b]
        t_rows = list(range(0, n + 1))  # target rows read by the statistics
        d_rows = [k for k in range(0, n + 1) if k < G]  # draft rows exist for positions < gamma
        want += len(t_rows) * V * 2 + len(d_rows) * V * 4
        want += G * 4 + (G + 1) * 4 + 4
    _, s2 = bench.sample_bytes(cfg, B, G, V, n_acc)
    assert bench.early_exit_bytes(cfg, B, G, V, n_acc) == want + s2
    # never more than the one-pass call
    s1, _ = bench.sample_bytes(cfg, B, G, V, n_acc)
    assert bench.early_exit_bytes(cfg, B, G, V, n_acc) <= s1 + s2
