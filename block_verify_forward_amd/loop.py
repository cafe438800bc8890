"""The DFlash speculative decoding loop over the C ABI ([CARD] "How it is used"; [PR2303] "What
changes", "Proof"): per round the draft proposes block - 1 tokens from the target's taps, the target
verifies [last token, proposals] in one batched pass, the greedy longest-prefix accept picks the
emitted tokens and commit_verify_rows keeps the rows on the accepted path.

Sequencing only: every step runs in the library's kernels on the models' stream; the host reads
the accepted count and the emitted tokens in one copy per round. The proposals are
written by the draft straight into the verify's token rows, the last emitted token is copied on the
device into row 0 of the next round, and the taps of the accepted rows become the draft's next
context rows without leaving the device.

Optional steering (seeded acceptance for synthetic weights): before the accept, row m < a gets a
large bonus on proposal m + 1 and row a a large penalty on proposal a + 1, so exactly a proposals
are accepted whatever the weights.

With a temperature above 0 every verify row is sampled ([CARD] "How it is used") through the
library's sampled accept: the Philox key is the loop's seed and the counter offset is the round
number, so a run is reproducible and every round draws fresh uniforms.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import bvf


class SpecLoop:
    def __init__(self, target: bvf.Model, draft: bvf.Model, block: int = 8, mask_token: Optional[int] = None,
                 embedding_scale: float = 1.0, steer_bonus: float = 1.0e4, temperature: float = 0.0, seed: int = 0):
        self.T, self.D = target, draft
        self.block = block
        m = target.m
        self.mask = m.vocab - 1 if mask_token is None else mask_token
        self.scale = embedding_scale
        self.bonus = steer_bonus
        dev = "cuda"
        self.toks = torch.zeros(block, dtype=torch.int32, device=dev)            # [last, d_1 .. d_{B-1}]
        self.logits = torch.empty((block, m.vocab), dtype=torch.float32, device=dev)
        self.taps = torch.empty((block, len(m.tap_layers), m.hidden), dtype=torch.int16, device=dev)
        # the emitted tokens and the accepted count side by side, so one copy to the host reads both
        self.res = torch.zeros(block + 1, dtype=torch.int32, device=dev)
        self.out = self.res[:block]
        self.n_acc = self.res[block:]
        self.add = torch.zeros(block - 1, dtype=torch.float32, device=dev)
        self.draws = torch.zeros(block, dtype=torch.int32, device=dev)
        self.temperature = float(temperature)
        self.seed = int(seed)
        self.n_rounds = 0
        self.n_new = 0

    def start(self, last_token: int):
        """The token the next round starts from (already in the target's context)."""
        self.toks[0] = int(last_token)
        self.n_new = 0

    def round(self, steer_a: Optional[int] = None):
        """One round; returns (accepted drafts a, emitted tokens [a + 1])."""
        B = self.block
        self.D.draft_block_forward(self.T, self.taps[: self.n_new] if self.n_new else None, self.n_new,
                                   self.toks[0:1], B, self.scale, self.mask, self.toks[1:], None)
        self.T.verify_batch(self.toks, self.logits, self.taps)
        if steer_a is not None:
            add = np.zeros(B - 1, dtype=np.float32)
            add[:steer_a] = self.bonus
            if steer_a < B - 1:
                add[steer_a] = -self.bonus
            self.add.copy_(torch.from_numpy(add))
            self.T.steer_logits(self.logits, self.toks[1:], self.add)
        if self.temperature > 0.0:
            self.T.accept_sampled(self.logits, self.toks, self.out, self.n_acc, self.temperature, self.seed,
                                  self.n_rounds, self.draws)
        else:
            self.T.accept_greedy(self.logits, self.toks, self.out, self.n_acc)
        self.n_rounds += 1
        res = self.res.cpu().numpy()   # one read of the round's results
        a = int(res[B])
        self.T.commit_verify_rows(a + 1)
        emitted = res[: a + 1].tolist()
        self.toks[0:1].copy_(self.out[a:a + 1])
        self.n_new = a + 1
        return a, emitted

    def run(self, n_tokens: int, steer: Optional[np.ndarray] = None) -> List[int]:
        """Rounds until at least n_tokens tokens are emitted; steer[i] is round i's accept length."""
        toks: List[int] = []
        self.accepted: List[int] = []
        i = 0
        while len(toks) < n_tokens:
            a, em = self.round(None if steer is None else int(steer[i]))
            self.accepted.append(a)
            toks.extend(em)
            i += 1
        return toks
