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

An iteration is some thirty small launches; ``capture`` records one iteration
(with the state carried over inside it) as a HIP graph, so that ``replay``
costs one launch from the host.
"""
from __future__ import annotations

import torch

from . import binding


def _rows(npos, B, V, dtype, device):
    """Position-major row buffer [npos][B][Vp] (Vp: V rounded up to 16 bytes)
    and its [B][npos][V] view. The verify reads the view through its strides;
    the gathers write whole [B][Vp] blocks of the buffer."""
    per = 16 // torch.tensor([], dtype=dtype).element_size()
    Vp = -(-V // per) * per
    buf = torch.empty((npos, B, Vp), dtype=dtype, device=device)
    return buf, buf.permute(1, 0, 2)[..., :V]


class MarkovLoop:
    def __init__(self, target_table: torch.Tensor, draft_table: torch.Tensor, gamma: int,
                 temperature: torch.Tensor):
        if target_table.shape != draft_table.shape or target_table.dim() != 2 or \
                target_table.shape[0] != target_table.shape[1]:
            raise ValueError("tables must both be [V][V]")
        self.V = target_table.shape[0]
        per = 16 // target_table.element_size()
        Vp = -(-self.V // per) * per
        if Vp != self.V:  # pad the tables' rows so a gathered row is a whole buffer row
            target_table = torch.nn.functional.pad(target_table, (0, Vp - self.V))
            draft_table = torch.nn.functional.pad(draft_table, (0, Vp - self.V))
        self.target, self.draft = target_table.contiguous(), draft_table.contiguous()
        self.gamma = int(gamma)
        self.T = temperature
        self.B = temperature.shape[0]
        dev = target_table.device
        B, G, V = self.B, self.gamma, self.V
        self.d_buf, self.d_rows = _rows(G, B, V, draft_table.dtype, dev)
        self.t_buf, self.t_rows = _rows(G + 1, B, V, target_table.dtype, dev)
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
        G, V = self.gamma, self.V
        prev = state
        for i in range(G):
            torch.index_select(self.draft, 0, prev, out=self.d_buf[i])
            binding.spec_draft_sample(self.d_buf[i][:, :V], u_draft[:, i].contiguous(), self.T,
                                      out_tokens=self.x_cols[i], workspace=self.ws_draft)
            prev = self.x_cols[i].long()
        self.x.copy_(self.x_cols.t())
        torch.index_select(self.target, 0, state, out=self.t_buf[0])
        torch.index_select(self.target, 0, self.x_cols.view(-1).long(), out=self.t_buf[1:].view(G * self.B, -1))
        binding.spec_verify_sample(self.t_rows, self.d_rows, self.x, u_verify, self.T, out_num_accepted=self.n,
                                   out_tokens=self.tokens, workspace=self.ws_verify)
        new_state = self.tokens.gather(1, self.n.clamp(min=0).long()[:, None])[:, 0]
        return self.n, self.tokens, new_state.long()

    def capture(self, state: torch.Tensor, u_draft: torch.Tensor, u_verify: torch.Tensor):
        """Record one iteration as a graph on static buffers initialised from
        the arguments (the first iteration is also run eagerly, to size every
        workspace before capture). The graph reads u_draft / u_verify from
        self.g_ud / self.g_uv and the state from self.g_state, and writes the
        next state back into self.g_state; outputs are self.n, self.tokens."""
        self.g_state = state.clone()
        self.g_ud = u_draft.clone()
        self.g_uv = u_verify.clone()
        self.step(self.g_state.clone(), self.g_ud, self.g_uv)  # eager warm-up: allocates workspaces
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            _, _, nxt = self.step(self.g_state, self.g_ud, self.g_uv)
            self.g_state.copy_(nxt)
        torch.cuda.synchronize()

    def replay(self, u_draft: torch.Tensor, u_verify: torch.Tensor):
        """One captured iteration with new uniforms; the state advances inside
        the graph. Returns (n, tokens) (overwritten by the next replay)."""
        self.g_ud.copy_(u_draft)
        self.g_uv.copy_(u_verify)
        self.graph.replay()
        return self.n, self.tokens
