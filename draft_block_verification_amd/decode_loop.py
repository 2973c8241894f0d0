"""A multi-step toy decode loop around the verify path, with fixed shapes for graph replay.

DSpark summary, "Architecture" (decode round: the drafter proposes a block, the
scheduler keeps its confident prefix, the target verifies the block in one pass,
accepts a prefix and adds its own token) and "Engineering" (the scheduler in
practice runs inside CUDA-graph replay with zero-overhead scheduling, the batch
of the next step fixed before the current one ends; variable-length requests
are flattened, not padded).

Toy models, so the loop runs without trained weights:

* target: a bigram model over the given LM head. The hidden state at a token is
  its row of an embedding table E (bf16 [V][d]); the target's next-token logits
  after token t are E[t] . W^T.
* drafter: a table. After token t it proposes draft_next[t] with conditional
  confidence draft_conf[t].

One step for every request: draft gamma tokens from the last emitted one,
gather the hidden rows of the block (last token and the gamma drafts), keep a
prefix (confidence threshold on the running product of the confidences, or the
prefix scheduler on the conditional confidences), verify greedily with
sd_verify_greedy, then append the accepted drafts and the target's token to
the request's output. Every operation is a device kernel on one stream with no
host synchronisation, so a whole step can be captured in a HIP graph.

The table lookups, gathers and appends are torch device ops (indexing and
elementwise only); the verify path itself is the library's.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


class ToyDecodeLoop:
    def __init__(self, lm_head, embed: torch.Tensor, draft_next: torch.Tensor,
                 draft_conf: torch.Tensor, B: int, gamma: int, max_steps: int,
                 threshold: float = 0.3, scheduler: Optional[int] = None,
                 sps: Optional[torch.Tensor] = None):
        V, d = embed.shape
        self.B, self.gamma, self.V, self.d = B, gamma, V, d
        self.max_steps = max_steps
        dev = embed.device
        self.lm_head, self.embed = lm_head, embed
        self.draft_next = draft_next.to(torch.int64)
        self.draft_conf = draft_conf.to(torch.float32)
        self.scheduler = scheduler
        self.vr = _lib.VerifyRound(B, gamma, d, V, 0.0, True, threshold, device=dev,
                                   scheduler=scheduler, sps=sps)
        # Output: at most gamma + 1 tokens per step, then one spare column that takes
        # the writes of positions past a request's accepted length.
        self.cap = max_steps * (gamma + 1) + 1
        self.out = torch.zeros((B, self.cap + 1), dtype=torch.int32, device=dev)
        self.length = torch.zeros(B, dtype=torch.int64, device=dev)
        self.last = torch.zeros(B, dtype=torch.int64, device=dev)
        self.draft_tokens = torch.zeros((B, gamma), dtype=torch.int32, device=dev)
        self.conf = torch.zeros((B, gamma), dtype=torch.float32, device=dev)
        # Conditional confidences of the last three steps (the asynchronous scheduler
        # sizes the batch from the ones of two steps before).
        self.cond = torch.zeros((3, B, gamma), dtype=torch.float32, device=dev)
        self.pos = torch.arange(gamma + 1, device=dev)

    def reset(self, start: torch.Tensor) -> None:
        """Start every request from its token in `start` (int [B]); the start token is
        the first output token."""
        self.out.zero_()
        self.out[:, 0] = start.to(torch.int32)
        self.length.fill_(1)
        self.last.copy_(start.to(torch.int64))
        self.cond.fill_(1.0)
        self.vr.counters.zero_()

    def step(self, slot: int) -> None:
        """One decode step; `slot` (0, 1, 2 in turn) picks the confidence history row."""
        B, g = self.B, self.gamma
        # Draft: x_1 .. x_g from the drafter table, conditional confidences alongside.
        x = self.last
        cond = self.cond[slot]
        for j in range(g):
            cond[:, j] = self.draft_conf[x]
            x = self.draft_next[x]
            self.draft_tokens[:, j] = x.to(torch.int32)
        # Block rows: the last token, then the drafts.
        block = torch.cat([self.last[:, None], self.draft_tokens.to(torch.int64)], dim=1)
        hidden = self.embed[block]                                   # [B][g + 1][d]
        if self.scheduler is None:
            run = torch.ones(B, dtype=torch.float32, device=cond.device)
            for j in range(g):                                       # survival = running product
                run = run * cond[:, j]
                self.conf[:, j] = run
            conf_in, stale = self.conf, None
        else:
            conf_in = cond
            stale = self.cond[(slot + 1) % 3] if self.scheduler == _lib.SCHED_TOP_K else None
        acc, nxt = self.vr.run(hidden, self.lm_head, self.draft_tokens, conf_in, conf_stale=stale)
        # Commit: accepted drafts x_1 .. x_a, then the target's token, at length[r] + i.
        a = acc.to(torch.int64)[:, None]
        vals = torch.where(self.pos[None, :] < a,
                           torch.cat([self.draft_tokens, self.draft_tokens[:, :1]], dim=1),
                           nxt.to(torch.int32)[:, None])
        idx = self.length[:, None] + self.pos[None, :]
        idx = torch.where((self.pos[None, :] <= a) & (idx < self.cap), idx,
                          torch.full_like(idx, self.cap))
        self.out.scatter_(1, idx, vals)
        self.length.add_(a[:, 0] + 1).clamp_(max=self.cap)
        self.last.copy_(nxt.to(torch.int64))

    def tokens(self):
        """Host copy of each request's output tokens."""
        out, length = self.out.cpu().numpy(), self.length.cpu().numpy()
        return [out[r, :length[r]].tolist() for r in range(self.B)]
