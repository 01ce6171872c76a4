"""spec_verify_sample_noalloc (no workspace: the library's static device array)
against spec_verify_sample (a caller's workspace) through the C ABI: two calls
in a row, the second with a smaller input, then configuration 5's full call.
Both entry points run the same kernels on the same decomposition, so their
outputs must agree bit for bit; each is also checked against the fp64 oracle
with the parity contract. A call too large for the array fails with a
ValueError (SV_ERR_SCRATCH) and leaves the next call unaffected."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _noalloc(gpu, tens):
    n, tok, d = gpu.spec_verify_sample_noalloc(**tens, diag=True)
    torch.cuda.synchronize()
    out = {"n": n.cpu().numpy(), "tokens": tok.cpu().numpy()}
    out.update({k: v.cpu().numpy() for k, v in d.items()})
    return out


def _same(a, b, name):
    for k in ("n", "tokens", "p_x", "q_x", "resid_mass"):
        assert np.array_equal(a[k], b[k], equal_nan=True), (name, k)


@pytest.mark.parametrize("first,second", [
    ((64, 4, 128256, "bf16", "bf16", 0.7), (6, 3, 20000, "bf16", "f32", 1.1)),
    ((40, 6, 50000, "f32", "f32", 1.0), (1, 2, 1000, "bf16", "bf16", 0.9)),
])
def test_noalloc_matches_workspace_call(gpu, first, second):
    for k, (B, G, V, tdt, ddt, T) in enumerate((first, second)):
        H.log(f"noalloc call {k + 1}: B={B} gamma={G} V={V} {tdt}/{ddt}")
        inp = synth.make_custom_sample(B, G, V, tdt, ddt, T=T, noise_sd=0.6, seed=100 + B + k)
        tens = H.sample_tensors(inp)
        ref = H.run_sample(gpu, tens)
        got = _noalloc(gpu, tens)
        _same(ref, got, f"call {k + 1}")
        t = H.check_sample(inp, got)
        H.log(f"[noalloc call {k + 1}] {t.summary()}")
        assert not t.fail, t.fail[:5]


def test_noalloc_full_config5_and_size_limit(gpu):
    inp = synth.make_sample_inputs(5, seed=0)
    tens = H.sample_tensors(inp)
    ref = H.run_sample(gpu, tens)
    got = _noalloc(gpu, tens)
    _same(ref, got, "config 5")
    # a call whose workspace exceeds the array: refused before any work, outputs untouched
    V = 128256
    big = {"target": torch.zeros((4096, 9, V), dtype=torch.bfloat16, device="cuda"),
           "draft": torch.zeros((4096, 8, V), dtype=torch.bfloat16, device="cuda"),
           "draft_tokens": torch.zeros((4096, 8), dtype=torch.int32, device="cuda"),
           "uniforms": torch.zeros((4096, 9), dtype=torch.float32, device="cuda"),
           "temperature": torch.ones(4096, dtype=torch.float32, device="cuda")}
    with pytest.raises(ValueError, match="static scratch"):
        gpu.spec_verify_sample_noalloc(**big)
    del big
    again = _noalloc(gpu, tens)
    _same(ref, again, "config 5 after a refused call")
