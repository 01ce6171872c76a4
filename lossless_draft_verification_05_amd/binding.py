"""ctypes binding of libspec_verify.so.

Argument marshalling only: every step of the verify path runs in the HIP
kernels behind the C ABI declared in include/spec_verify.h. PyTorch supplies
device memory and the current stream; nothing here computes on the data.
There is no fallback: if the shared library is missing, ``load`` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; SV_LIBRARY may name another build of the same library.
LIB_PATH = os.environ.get("SV_LIBRARY") or os.path.join(HERE, "libspec_verify.so")

SV_F32, SV_BF16 = 0, 1
SV_OK = 0
_ARG_ERRORS = {-1, -2, -3, -4, -5, -7, -8}

_lib = None

# Every symbol the header declares, with its ctypes signature.
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "sv_sample_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "sv_tree_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "spec_verify_sample": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _i32,
                                  _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_sample_stage": (_i32, [_i32, _vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _i32,
                                        _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_sample_early_exit": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _i32, _i32,
                                             _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_sample_noalloc": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _i32, _i32,
                                          _i32, _vp, _vp, _vp, _vp]),
    "spec_verify_sample_early_exit_grouped": (_i32, [_i32, _vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _vp,
                                                     _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_greedy_tree": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                       _sz, _vp]),
    "spec_verify_greedy_tree_stage": (_i32, [_i32, _vp, _i32, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp,
                                             _vp, _vp, _sz, _vp]),
    "sv_draft_workspace_bytes": (_sz, [_i32, _i32]),
    "spec_draft_sample": (_i32, [_vp, _i32, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "spec_draft_sample_stage": (_i32, [_i32, _vp, _i32, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "spec_tree_mask": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "sv_status_string": (ctypes.c_char_p, [_i32]),
    "sv_last_hip_error": (_i32, []),
    "sv_version": (ctypes.c_char_p, []),
}


class SampleDiag(ctypes.Structure):
    _fields_ = [("p_x", ctypes.c_void_p), ("q_x", ctypes.c_void_p), ("resid_mass", ctypes.c_void_p)]


def load(path: str = LIB_PATH):
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m lossless_draft_verification_05_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(st: int) -> str:
    return load().sv_status_string(st).decode()


def _check(st: int, what: str):
    if st == SV_OK:
        return
    msg = f"{what}: {status_string(st)} (status {st})"
    if st in _ARG_ERRORS:
        raise ValueError(msg)
    raise RuntimeError(f"{msg}; hipError {load().sv_last_hip_error()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise ValueError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _stream_obj(stream, device):
    return stream if stream is not None else torch.cuda.current_stream(device)


def _need(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _logits3(t: torch.Tensor, name: str, rows: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 3:
        raise ValueError(f"{name} must be a 3-d CUDA tensor")
    if t.shape[1] != rows:
        raise ValueError(f"{name} must have {rows} rows per sequence, got {t.shape[1]}")
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError(f"{name} rows must be contiguous (last stride 1)")
    return t.stride(0), t.stride(1)


class Workspace:
    """Device workspace grown on demand and reused by calls.

    The kernels keep nothing in it between calls and need it uninitialised;
    calls that may run at the same time need separate Workspace objects. The
    buffer is allocated on the stream of the call that grows it; a call on any
    other stream records that stream on the buffer (record_stream), so the
    caching allocator never hands the memory out again while such a call may
    still use it, also after the buffer is replaced by a larger one.
    """

    def __init__(self):
        self.buf = None
        self._alloc_stream = None

    def get(self, nbytes: int, device, stream=None) -> torch.Tensor:
        s = _stream_obj(stream, device)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            with torch.cuda.stream(s):
                self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._alloc_stream = s
        elif s != self._alloc_stream:
            self.buf.record_stream(s)
        return self.buf


# Default workspaces, one per (device, stream): calls on different streams never
# share one, so they can overlap.
_default_ws = {}


def _workspace(ws, nbytes, device, stream=None):
    """A Workspace object (default: one per device and stream) or a caller-managed uint8 tensor."""
    if ws is None:
        s = _stream_obj(stream, device)
        ws = _default_ws.setdefault((device, s.cuda_stream), Workspace())
    buf = ws.get(nbytes, device, stream) if isinstance(ws, Workspace) else ws
    if buf.numel() < nbytes:
        raise ValueError(f"workspace has {buf.numel()} bytes, needs {nbytes}")
    return buf


class Prepared:
    """A call whose arguments were checked and marshalled once. Calling it
    enqueues the same kernels again, on the same tensors and stream (a serving
    loop's fixed buffers), with no per-call Python checks; it returns the same
    outputs as the call it was prepared from. It keeps its tensors alive."""

    __slots__ = ("_cfn", "_args", "_name", "outputs", "_keep")

    def __init__(self, cfn, args, name, outputs, keep):
        self._cfn, self._args, self._name, self.outputs, self._keep = cfn, args, name, outputs, keep

    def __call__(self):
        _check(self._cfn(*self._args), self._name)
        return self.outputs


def _launch(cfn, args, name, outputs, keep, prepare):
    call = Prepared(cfn, args, name, outputs, keep)
    return call if prepare else call()


def sv_sample_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return int(load().sv_sample_workspace_bytes(B, gamma, V))


def sv_tree_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(load().sv_tree_workspace_bytes(B, N, V))


def _sample_call(stage, target, draft, draft_tokens, uniforms, temperature, out_num_accepted, out_tokens, diag,
                 workspace, stream, prepare=False):
    lib = load()
    B, G1, V = target.shape
    G = G1 - 1
    ts, tr = _logits3(target, "target", G + 1)
    ds, dr = _logits3(draft, "draft", G)
    if draft.shape[0] != B or draft.shape[2] != V:
        raise ValueError("draft must be [B][gamma][V] matching target")
    dev = target.device
    _need(draft_tokens, "draft_tokens", torch.int32, (B, G))
    _need(uniforms, "uniforms", torch.float32, (B, G + 1))
    _need(temperature, "temperature", torch.float32, (B,))
    if out_num_accepted is None:
        out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    _need(out_num_accepted, "out_num_accepted", torch.int32, (B,))
    _need(out_tokens, "out_tokens", torch.int32, (B, G + 1))
    d = None
    dptr = None
    if diag:
        d = {"p_x": torch.empty((B, G), dtype=torch.float32, device=dev),
             "q_x": torch.empty((B, G), dtype=torch.float32, device=dev),
             "resid_mass": torch.empty(B, dtype=torch.float32, device=dev)}
        dptr = SampleDiag(d["p_x"].data_ptr(), d["q_x"].data_ptr(), d["resid_mass"].data_ptr())
    nbytes = sv_sample_workspace_bytes(B, G, V)
    if nbytes == 0:
        raise ValueError(f"shape B={B} gamma={G} V={V} out of range")
    outputs = (out_num_accepted, out_tokens, d)
    if stage == "noalloc":  # no workspace: the library's static array
        args = (_ptr(target), _dtype_code(target), ts, tr, _ptr(draft), _dtype_code(draft), ds, dr,
                _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), B, G, V, _ptr(out_num_accepted),
                _ptr(out_tokens), ctypes.byref(dptr) if dptr is not None else None, _stream(stream))
        keep = (target, draft, draft_tokens, uniforms, temperature, d, dptr)
        return _launch(lib.spec_verify_sample_noalloc, args, "spec_verify_sample_noalloc", outputs, keep, prepare)
    ws = _workspace(workspace, nbytes, dev, stream)
    args = (_ptr(target), _dtype_code(target), ts, tr, _ptr(draft), _dtype_code(draft), ds, dr, _ptr(draft_tokens),
            _ptr(uniforms), _ptr(temperature), B, G, V, _ptr(out_num_accepted), _ptr(out_tokens),
            ctypes.byref(dptr) if dptr is not None else None, _ptr(ws), ws.numel(), _stream(stream))
    keep = (target, draft, draft_tokens, uniforms, temperature, ws, d, dptr)
    if stage is None:
        return _launch(lib.spec_verify_sample, args, "spec_verify_sample", outputs, keep, prepare)
    if stage == "early_exit":
        return _launch(lib.spec_verify_sample_early_exit, args, "spec_verify_sample_early_exit", outputs, keep,
                       prepare)
    if isinstance(stage, tuple):  # ("early_exit", tail_start)
        return _launch(lib.spec_verify_sample_early_exit_grouped, (int(stage[1]),) + args,
                       f"spec_verify_sample_early_exit_grouped({stage[1]})", outputs, keep, prepare)
    return _launch(lib.spec_verify_sample_stage, (stage,) + args, f"spec_verify_sample_stage({stage})", outputs,
                   keep, prepare)


def spec_verify_sample(target, draft, draft_tokens, uniforms, temperature, *, out_num_accepted=None,
                       out_tokens=None, diag=False, workspace=None, stream=None, prepare=False):
    """Speculative-sampling verify of B sequences on the GPU (see include/spec_verify.h).

    target [B][gamma+1][V] and draft [B][gamma][V] are bf16 or fp32 CUDA tensors
    whose rows are contiguous and 16-byte aligned (a stride-0 batch dimension
    is allowed); draft_tokens int32 [B][gamma]; uniforms fp32 [B][gamma+1];
    temperature fp32 [B]. Returns (num_accepted [B], tokens [B][gamma+1], diag
    dict or None). Work is enqueued on ``stream`` (default: current stream).
    With ``prepare=True`` nothing is enqueued: the result is a Prepared call
    that enqueues the work each time it is called. (The same holds for every
    entry point below.)
    """
    return _sample_call(None, target, draft, draft_tokens, uniforms, temperature, out_num_accepted, out_tokens,
                        diag, workspace, stream, prepare)


def spec_verify_sample_noalloc(target, draft, draft_tokens, uniforms, temperature, *, out_num_accepted=None,
                               out_tokens=None, diag=False, stream=None, prepare=False):
    """spec_verify_sample without a workspace: the library uses its static device array
    (SV_NOALLOC_SCRATCH_BYTES per GPU) and allocates nothing; calls on one GPU must not
    overlap. Outputs are allocated here unless given (pass them to allocate nothing at all)."""
    return _sample_call("noalloc", target, draft, draft_tokens, uniforms, temperature, out_num_accepted, out_tokens,
                        diag, None, stream, prepare)


def spec_verify_sample_early_exit(target, draft, draft_tokens, uniforms, temperature, *, out_num_accepted=None,
                                  out_tokens=None, diag=False, workspace=None, stream=None, prepare=False):
    """spec_verify_sample that reads no row after a sequence's first rejection: same arguments and
    outputs (diag p_x, q_x are NaN after the first rejection)."""
    return _sample_call("early_exit", target, draft, draft_tokens, uniforms, temperature, out_num_accepted,
                        out_tokens, diag, workspace, stream, prepare)


def spec_verify_sample_early_exit_grouped(tail_start, target, draft, draft_tokens, uniforms, temperature, *,
                                          out_num_accepted=None, out_tokens=None, diag=False, workspace=None,
                                          stream=None, prepare=False):
    """spec_verify_sample_early_exit with the grouping chosen by the caller: positions
    0..tail_start-1 get a statistics launch each, tail_start..gamma share one (tail_start < 0:
    chosen from the sizes)."""
    return _sample_call(("early_exit", int(tail_start)), target, draft, draft_tokens, uniforms, temperature,
                        out_num_accepted, out_tokens, diag, workspace, stream, prepare)


def spec_verify_sample_stage(stage, target, draft, draft_tokens, uniforms, temperature, *, out_num_accepted=None,
                             out_tokens=None, diag=False, workspace=None, stream=None, prepare=False):
    """One stage of spec_verify_sample: 1 row statistics, 2 accept tests + residual/bonus draw + outputs,
    3 the reads of stage 1 alone (a measurement of its read rate; no outputs)."""
    return _sample_call(int(stage), target, draft, draft_tokens, uniforms, temperature, out_num_accepted,
                        out_tokens, diag, workspace, stream, prepare)


def spec_draft_sample(logits, uniforms, temperature, *, out_tokens=None, want_prob=False, workspace=None,
                      stream=None, stage=None, prepare=False):
    """Draft-side sampler (see include/spec_verify.h): one token per row of logits [B][V] (bf16 or fp32,
    contiguous 16-byte aligned rows) from softmax(row / T) at the row's uniform. Returns (tokens [B] int32,
    q(token) [B] float32 or None). ``stage`` 1 or 2 runs one of its two kernels."""
    lib = load()
    if not isinstance(logits, torch.Tensor) or not logits.is_cuda or logits.dim() != 2:
        raise ValueError("logits must be a 2-d CUDA tensor [B][V]")
    B, V = logits.shape
    if logits.stride(1) != 1 and V > 1:
        raise ValueError("logits rows must be contiguous (last stride 1)")
    dev = logits.device
    _need(uniforms, "uniforms", torch.float32, (B,))
    _need(temperature, "temperature", torch.float32, (B,))
    if out_tokens is None:
        out_tokens = torch.empty(B, dtype=torch.int32, device=dev)
    _need(out_tokens, "out_tokens", torch.int32, (B,))
    prob = torch.empty(B, dtype=torch.float32, device=dev) if want_prob else None
    nbytes = int(lib.sv_draft_workspace_bytes(B, V))
    if nbytes == 0:
        raise ValueError(f"shape B={B} V={V} out of range")
    ws = _workspace(workspace, nbytes, dev, stream)
    args = (_ptr(logits), _dtype_code(logits), logits.stride(0), _ptr(uniforms), _ptr(temperature), B, V,
            _ptr(out_tokens), _ptr(prob) if prob is not None else None, _ptr(ws), ws.numel(), _stream(stream))
    keep = (logits, uniforms, temperature, ws)
    if stage is None:
        return _launch(lib.spec_draft_sample, args, "spec_draft_sample", (out_tokens, prob), keep, prepare)
    return _launch(lib.spec_draft_sample_stage, (int(stage),) + args, f"spec_draft_sample_stage({stage})",
                   (out_tokens, prob), keep, prepare)


def _tree_call(stage, logits, parents, tokens, out_accept_len, out_path, out_bonus, out_argmax, want_argmax,
               workspace, stream, prepare=False):
    lib = load()
    B, N, V = logits.shape
    s0, s1 = _logits3(logits, "logits", N)
    dev = logits.device
    _need(parents, "parents", torch.int32, (B, N))
    _need(tokens, "tokens", torch.int32, (B, N))
    if out_accept_len is None:
        out_accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_path is None:
        out_path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if out_bonus is None:
        out_bonus = torch.empty(B, dtype=torch.int32, device=dev)
    if out_argmax is None and want_argmax:
        out_argmax = torch.empty((B, N), dtype=torch.int32, device=dev)
    nbytes = sv_tree_workspace_bytes(B, N, V)
    if nbytes == 0:
        raise ValueError(f"shape B={B} N={N} V={V} out of range")
    ws = _workspace(workspace, nbytes, dev, stream)
    args = (_ptr(logits), _dtype_code(logits), s0, s1, _ptr(parents), _ptr(tokens), B, N, V, _ptr(out_accept_len),
            _ptr(out_path), _ptr(out_bonus), _ptr(out_argmax), _ptr(ws), ws.numel(), _stream(stream))
    keep = (logits, parents, tokens, ws)
    outputs = (out_accept_len, out_path, out_bonus, out_argmax)
    if stage is None:
        return _launch(lib.spec_verify_greedy_tree, args, "spec_verify_greedy_tree", outputs, keep, prepare)
    return _launch(lib.spec_verify_greedy_tree_stage, (stage,) + args, f"spec_verify_greedy_tree_stage({stage})",
                   outputs, keep, prepare)


def spec_verify_greedy_tree(logits, parents, tokens, *, out_accept_len=None, out_path=None, out_bonus=None,
                            out_argmax=None, want_argmax=True, workspace=None, stream=None, prepare=False):
    """Greedy decoding-tree verify of B trees (see include/spec_verify.h).

    logits [B][N][V] bf16/fp32 (rows contiguous, 16-byte aligned); parents and
    tokens int32 [B][N]. Returns (accept_len [B], path [B][N], bonus [B],
    argmax [B][N] or None).
    """
    return _tree_call(None, logits, parents, tokens, out_accept_len, out_path, out_bonus, out_argmax, want_argmax,
                      workspace, stream, prepare)


def spec_verify_greedy_tree_stage(stage, logits, parents, tokens, *, out_accept_len=None, out_path=None,
                                  out_bonus=None, out_argmax=None, want_argmax=True, workspace=None, stream=None,
                                  prepare=False):
    """One stage of spec_verify_greedy_tree: 1 per-row argmax, 2 tree resolve and outputs."""
    return _tree_call(int(stage), logits, parents, tokens, out_accept_len, out_path, out_bonus, out_argmax,
                      want_argmax, workspace, stream, prepare)


def version() -> str:
    return load().sv_version().decode()


def spec_tree_mask(parents, blocks=None, *, want_mask=True, want_relaxed=False, want_depth=True, out_mask=None,
                   out_relaxed=None, out_depth=None, stream=None, prepare=False):
    """Tree-attention masks of B draft trees (see include/spec_verify.h). parents [B][N] int32 (and blocks
    [B][N] int32 for the relaxed mask). Returns (mask uint8 [B][N][N] or None, relaxed or None, depth int32
    [B][N] or None)."""
    lib = load()
    if not isinstance(parents, torch.Tensor) or parents.dim() != 2:
        raise ValueError("parents must be a 2-d tensor [B][N]")
    B, N = parents.shape
    dev = parents.device
    _need(parents, "parents", torch.int32, (B, N))
    if blocks is not None:
        _need(blocks, "blocks", torch.int32, (B, N))
    if want_mask and out_mask is None:
        out_mask = torch.empty((B, N, N), dtype=torch.uint8, device=dev)
    if want_relaxed and out_relaxed is None:
        out_relaxed = torch.empty((B, N, N), dtype=torch.uint8, device=dev)
    if want_depth and out_depth is None:
        out_depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    for t, name in ((out_mask, "out_mask"), (out_relaxed, "out_relaxed")):
        if t is not None:
            _need(t, name, torch.uint8, (B, N, N))
    if out_depth is not None:
        _need(out_depth, "out_depth", torch.int32, (B, N))
    args = (_ptr(parents), _ptr(blocks), B, N, _ptr(out_mask), _ptr(out_relaxed), _ptr(out_depth), _stream(stream))
    return _launch(lib.spec_tree_mask, args, "spec_tree_mask", (out_mask, out_relaxed, out_depth), (parents, blocks),
                   prepare)
