"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

from lossless_draft_verification_05_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:sv|spec)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libspec_verify.so is not built (run python -m lossless_draft_verification_05_amd.build)")
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.SIGNATURES), set(names) ^ set(binding.SIGNATURES)


def test_version_and_status_strings(lib):
    assert b"spec_verify" in lib.sv_version()
    for st in range(-8, 1):
        assert lib.sv_status_string(st) and lib.sv_status_string(st) != b"unknown status"
    assert lib.sv_status_string(-99) == b"unknown status"
    assert lib.sv_last_hip_error() == 0


def test_workspace_sizes(lib):
    assert lib.sv_sample_workspace_bytes(0, 4, 32) == 0
    assert lib.sv_sample_workspace_bytes(1, 65, 32) == 0
    assert lib.sv_sample_workspace_bytes(1, 4, 0) == 0
    assert lib.sv_tree_workspace_bytes(1, 1025, 32) == 0
    a = lib.sv_sample_workspace_bytes(64, 4, 32000)
    b = lib.sv_sample_workspace_bytes(128, 4, 32000)
    c = lib.sv_sample_workspace_bytes(64, 4, 64000)
    assert 0 < a < b and a < c and a % 256 == 0
    assert lib.sv_tree_workspace_bytes(32, 60, 32000) > 0


# Fake device addresses: never dereferenced, because every case below fails validation.
A = 0x7F0000000000


def sample_args(**over):
    a = dict(target=A, tdt=1, tss=5 * 64, trs=64, draft=A + 0x100000, ddt=1, dss=4 * 64, drs=64, tokens=A + 0x200000,
             uniforms=A + 0x300000, temps=A + 0x400000, B=4, G=4, V=64, out_n=A + 0x500000, out_tok=A + 0x600000,
             diag=None, ws=A + 0x700000, wsb=1 << 30, stream=None)
    a.update(over)
    return a


def call_sample(lib, stage=None, **over):
    a = sample_args(**over)
    args = [a["target"], a["tdt"], a["tss"], a["trs"], a["draft"], a["ddt"], a["dss"], a["drs"], a["tokens"],
            a["uniforms"], a["temps"], a["B"], a["G"], a["V"], a["out_n"], a["out_tok"], a["diag"], a["ws"], a["wsb"],
            a["stream"]]
    if stage is None:
        return lib.spec_verify_sample(*args)
    if stage == "early_exit":
        return lib.spec_verify_sample_early_exit(*args)
    if stage == "grouped":
        return lib.spec_verify_sample_early_exit_grouped(1, *args)
    return lib.spec_verify_sample_stage(stage, *args)


@pytest.mark.parametrize("over,want", [
    (dict(target=None), -1), (dict(draft=None), -1), (dict(tokens=None), -1), (dict(uniforms=None), -1),
    (dict(temps=None), -1), (dict(out_n=None), -1), (dict(out_tok=None), -1),
    (dict(tdt=2), -3), (dict(ddt=-1), -3),
    (dict(B=0), -2), (dict(G=0), -2), (dict(G=65), -2), (dict(V=0), -2), (dict(V=(1 << 30) + 1), -2),
    (dict(trs=63), -2), (dict(drs=10), -2), (dict(tss=-8), -2),
    (dict(target=A + 2), -4), (dict(trs=68), -4), (dict(tss=5 * 64 + 4), -4), (dict(ddt=0, drs=66), -4),
    (dict(tokens=A + 2), -4), (dict(out_tok=A + 1), -4),
    (dict(ws=None), -5), (dict(wsb=100), -5), (dict(ws=A + 0x700010), -4),
    (dict(tss=1 << 60), -2),
])
def test_sample_argument_errors(lib, over, want):
    assert call_sample(lib, **over) == want
    for stage in (1, 2, 3, "early_exit", "grouped"):
        assert call_sample(lib, stage=stage, **over) == want


def call_noalloc(lib, **over):
    a = sample_args(**over)
    return lib.spec_verify_sample_noalloc(a["target"], a["tdt"], a["tss"], a["trs"], a["draft"], a["ddt"], a["dss"],
                                          a["drs"], a["tokens"], a["uniforms"], a["temps"], a["B"], a["G"], a["V"],
                                          a["out_n"], a["out_tok"], a["diag"], a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(target=None), -1), (dict(draft=None), -1), (dict(tokens=None), -1), (dict(uniforms=None), -1),
    (dict(temps=None), -1), (dict(out_n=None), -1), (dict(out_tok=None), -1),
    (dict(tdt=2), -3), (dict(ddt=-1), -3),
    (dict(B=0), -2), (dict(G=0), -2), (dict(G=65), -2), (dict(V=0), -2), (dict(V=(1 << 30) + 1), -2),
    (dict(trs=63), -2), (dict(tss=-8), -2),
    (dict(target=A + 2), -4), (dict(trs=68), -4), (dict(tokens=A + 2), -4), (dict(out_tok=A + 1), -4),
])
def test_noalloc_argument_errors(lib, over, want):
    """The entry point without a workspace checks the same arguments, before any HIP call."""
    assert call_noalloc(lib, **over) == want


def test_noalloc_size_limit(lib):
    """Configuration 5's call fits the 32 MiB static array; a call whose
    workspace would exceed it is refused with SV_ERR_SCRATCH before any HIP call."""
    assert 0 < lib.sv_sample_workspace_bytes(512, 5, 256000) <= 32 << 20
    V = 128256
    big = dict(B=4096, G=8, V=V, tss=9 * V, trs=V, dss=8 * V, drs=V)
    assert lib.sv_sample_workspace_bytes(4096, 8, V) > 32 << 20
    assert call_noalloc(lib, **big) == -8
    assert b"32 MiB" in lib.sv_status_string(-8)
    assert lib.sv_last_hip_error() == 0


def test_grouping_beyond_gamma(lib):
    a = sample_args()
    args = [a["target"], a["tdt"], a["tss"], a["trs"], a["draft"], a["ddt"], a["dss"], a["drs"], a["tokens"],
            a["uniforms"], a["temps"], a["B"], a["G"], a["V"], a["out_n"], a["out_tok"], a["diag"], a["ws"], a["wsb"],
            a["stream"]]
    assert lib.spec_verify_sample_early_exit_grouped(a["G"] + 1, *args) == -7
    bad = list(args)
    bad[0] = None
    assert lib.spec_verify_sample_early_exit_grouped(a["G"] + 1, *bad) == -1  # argument errors first


def test_unknown_stage(lib):
    assert call_sample(lib, stage=4) == -7
    assert call_sample(lib, stage=0) == -7
    assert call_sample(lib, stage=-1) == -7
    assert call_sample(lib, stage=-1) == -7


def call_tree(lib, **over):
    a = dict(logits=A, dt=1, ss=60 * 64, rs=64, parents=A + 0x100000, tokens=A + 0x200000, B=2, N=60, V=64,
             ol=A + 0x300000, op=A + 0x400000, ob=A + 0x500000, oa=None, ws=A + 0x600000, wsb=1 << 30, stream=None)
    a.update(over)
    return lib.spec_verify_greedy_tree(a["logits"], a["dt"], a["ss"], a["rs"], a["parents"], a["tokens"], a["B"],
                                       a["N"], a["V"], a["ol"], a["op"], a["ob"], a["oa"], a["ws"], a["wsb"],
                                       a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(logits=None), -1), (dict(parents=None), -1), (dict(tokens=None), -1), (dict(ol=None), -1),
    (dict(op=None), -1), (dict(ob=None), -1), (dict(dt=5), -3), (dict(N=0), -2), (dict(N=1025), -2),
    (dict(B=0), -2), (dict(rs=32), -2), (dict(logits=A + 8), -4), (dict(rs=68), -4), (dict(oa=A + 2), -4),
    (dict(ws=None), -5), (dict(wsb=16), -5),
])
def test_tree_argument_errors(lib, over, want):
    assert call_tree(lib, **over) == want


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        binding_mod = __import__("lossless_draft_verification_05_amd.binding", fromlist=["load"])
        saved = binding_mod._lib
        try:
            binding_mod._lib = None
            binding_mod.load(str(tmp_path / "missing.so"))
        finally:
            binding_mod._lib = saved


def test_tree_unknown_stage(lib):
    A0 = 0x7F0000000000
    args = [A0, 1, 60 * 64, 64, A0 + 0x100000, A0 + 0x200000, 2, 60, 64, A0 + 0x300000, A0 + 0x400000,
            A0 + 0x500000, None, A0 + 0x600000, 1 << 30, None]
    assert lib.spec_verify_greedy_tree_stage(0, *args) == -7
    assert lib.spec_verify_greedy_tree_stage(3, *args) == -7
    bad = list(args)
    bad[0] = None
    assert lib.spec_verify_greedy_tree_stage(1, *bad) == -1


def call_draft(lib, stage=None, **over):
    A = 0x10000000
    a = dict(logits=A, dt=0, rs=1024, uniforms=A + 0x800000, temps=A + 0x900000, B=4, V=1000,
             out=A + 0xA00000, prob=A + 0xB00000, ws=A + 0xC00000, wsb=1 << 24, stream=None)
    a.update(over)
    args = [a["logits"], a["dt"], a["rs"], a["uniforms"], a["temps"], a["B"], a["V"], a["out"], a["prob"], a["ws"],
            a["wsb"], a["stream"]]
    if stage is None:
        return lib.spec_draft_sample(*args)
    return lib.spec_draft_sample_stage(stage, *args)


@pytest.mark.parametrize("over,want", [
    (dict(logits=None), -1), (dict(uniforms=None), -1), (dict(temps=None), -1), (dict(out=None), -1),
    (dict(dt=2), -3), (dict(B=0), -2), (dict(V=0), -2), (dict(rs=999), -2), (dict(V=(1 << 30) + 1), -2),
    (dict(logits=0x10000002), -4), (dict(rs=1026), -4), (dict(out=0x10A00002), -4), (dict(prob=0x10B00001), -4),
    (dict(ws=None), -5), (dict(wsb=100), -5), (dict(ws=0x10C00010), -4),
])
def test_draft_argument_errors(lib, over, want):
    assert call_draft(lib, **over) == want
    for stage in (1, 2):
        assert call_draft(lib, stage=stage, **over) == want


def test_draft_unknown_stage_and_workspace_query(lib):
    assert call_draft(lib, stage=3) == -7 and call_draft(lib, stage=0) == -7
    assert lib.sv_draft_workspace_bytes(0, 10) == 0 and lib.sv_draft_workspace_bytes(4, 0) == 0
    assert lib.sv_draft_workspace_bytes(4, 1000) > 0


def test_tree_mask_argument_errors(lib):
    A = 0x10000000
    f = lib.spec_tree_mask
    assert f(None, None, 2, 5, A, None, None, None) == -1             # parents NULL
    assert f(A, None, 2, 5, A, A + 0x1000, None, None) == -1          # relaxed without blocks
    assert f(A, None, 0, 5, A, None, None, None) == -2                # B = 0
    assert f(A, None, 2, 0, A, None, None, None) == -2                # N = 0
    assert f(A, None, 2, 1025, A, None, None, None) == -2             # N too large
    assert f(A + 2, None, 2, 5, A, None, None, None) == -4            # parents misaligned
    assert f(A, A + 1, 2, 5, A, A + 0x1000, None, None) == -4         # blocks misaligned
    assert f(A, None, 2, 5, None, None, A + 0x2002, None) == -4       # depth misaligned
    assert f(A, None, 2, 5, None, None, None, None) == 0              # nothing requested: no launch


def test_argument_checks_from_many_threads(lib):
    """The host side keeps no shared mutable state: argument checks called
    from eight threads at once (ctypes releases the interpreter lock during
    each call) return the same statuses as one thread."""
    import threading

    cases = [(dict(target=None), -1), (dict(tdt=2), -3), (dict(B=0), -2), (dict(target=A + 2), -4),
             (dict(wsb=100), -5), (dict(G=65), -2)]
    errors = []

    def worker(k):
        try:
            for it in range(400):
                over, want = cases[(k + it) % len(cases)]
                got = call_sample(lib, **over)
                if got != want:
                    errors.append((k, it, over, got, want))
                if lib.sv_sample_workspace_bytes(64, 4, 32000) != lib.sv_sample_workspace_bytes(64, 4, 32000):
                    errors.append((k, it, "workspace size"))
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]
    assert lib.sv_last_hip_error() == 0
