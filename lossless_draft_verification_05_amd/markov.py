"""End-to-end speculative decoding on a synthetic Markov-chain model pair.

The 'models' are next-token logit tables: row s of a [V][V] table holds the
logits after token s, for the target and for a perturbed draft. One iteration
of the loop runs the method of [SD] ("The pith", "What carries the argument")
for B independent chains: the draft proposes gamma tokens one at a time
(spec_draft_sample on the draft row after each previous token), the target
rows after the current token and after each draft are gathered (the target's
one parallel pass), and spec_verify_sample keeps the accepted prefix and one
corrected or bonus token. The emitted stream of every chain must then be a
Markov chain with the target's tempered transition law ([SD] abstract, "Core
claim": exact samples of the target, across any number of calls).

Every step of the method runs in the library's kernels; torch provides the
tables, the row gathers (the stand-in for the models' forward passes) and the
buffers. Random numbers are inputs: u_draft [B][gamma] for the draft draws,
u_verify [B][gamma+1] for the accept tests and the final draw.
"""
from __future__ import annotations

import torch

from . import binding


def _padded(shape, V, dtype, device):
    """[..., V] view of a buffer whose rows are a multiple of 16 bytes long."""
    per = 16 // torch.tensor([], dtype=dtype).element_size()
    Vp = -(-V // per) * per
    return torch.empty(tuple(shape) + (Vp,), dtype=dtype, device=device)[..., :V]


class MarkovLoop:
    def __init__(self, target_table: torch.Tensor, draft_table: torch.Tensor, gamma: int,
                 temperature: torch.Tensor):
        if target_table.shape != draft_table.shape or target_table.dim() != 2 or \
                target_table.shape[0] != target_table.shape[1]:
            raise ValueError("tables must both be [V][V]")
        self.target, self.draft = target_table, draft_table
        self.V = target_table.shape[0]
        self.gamma = int(gamma)
        self.T = temperature
        self.B = temperature.shape[0]
        dev = target_table.device
        B, G, V = self.B, self.gamma, self.V
        self.d_rows = _padded((B, G), V, draft_table.dtype, dev)
        self.t_rows = _padded((B, G + 1), V, target_table.dtype, dev)
        self.x_cols = torch.empty((G, B), dtype=torch.int32, device=dev)  # x_i of every chain, per position
        self.x = torch.empty((B, G), dtype=torch.int32, device=dev)
        self.n = torch.empty(B, dtype=torch.int32, device=dev)
        self.tokens = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
        self.ws_draft = binding.Workspace()
        self.ws_verify = binding.Workspace()

    def step(self, state: torch.Tensor, u_draft: torch.Tensor, u_verify: torch.Tensor):
        """One speculative iteration from the last token `state` [B] (int64) of
        every chain. Returns (n [B], tokens [B][gamma+1], new_state [B]); the
        emitted tokens of chain b are tokens[b, :n[b] + 1]. Enqueued on the
        current stream; nothing synchronises."""
        prev = state
        for i in range(self.gamma):
            self.d_rows[:, i].copy_(self.draft.index_select(0, prev))
            binding.spec_draft_sample(self.d_rows[:, i], u_draft[:, i].contiguous(), self.T,
                                      out_tokens=self.x_cols[i], workspace=self.ws_draft)
            prev = self.x_cols[i].long()
        self.x.copy_(self.x_cols.t())
        self.t_rows[:, 0].copy_(self.target.index_select(0, state))
        self.t_rows[:, 1:].copy_(self.target[self.x.long()])
        binding.spec_verify_sample(self.t_rows, self.d_rows, self.x, u_verify, self.T, out_num_accepted=self.n,
                                   out_tokens=self.tokens, workspace=self.ws_verify)
        new_state = self.tokens.gather(1, self.n.clamp(min=0).long()[:, None])[:, 0]
        return self.n, self.tokens, new_state.long()
