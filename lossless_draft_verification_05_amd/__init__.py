"""MI355X-native verify step of speculative decoding (speculative sampling and
greedy decoding-tree verification) over hand-written gfx950 HIP kernels.

The C ABI is include/spec_verify.h (libspec_verify.so, built in-tree by
``python -m lossless_draft_verification_05_amd.build``); ``binding`` is its thin
ctypes wrapper. Importing this package does not load the library; the first
call does, and fails loudly if the library is missing.
"""


def __getattr__(name):
    if name in ("spec_verify_sample", "spec_verify_sample_stage", "spec_verify_sample_early_exit", "spec_draft_sample",
                "spec_verify_greedy_tree",
                "spec_verify_greedy_tree_stage", "spec_tree_mask",
                "sv_sample_workspace_bytes", "sv_tree_workspace_bytes", "Workspace"):
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
