"""Speculative decoding loop with a block drafter and greedy verification.

TEST INFRASTRUCTURE (see ``oracle/dflash.py``).  Written from the "DFlash"
technical summary: §1 (the drafter proposes, the target verifies in
parallel), §2.2 (features from the target's prefill feed the drafter's KV
cache; one block per forward pass), §2.3 (the block starts at a clean token the
target produced), §4/§5 (the output is lossless with respect to greedy
decoding).

Per cycle, with n committed tokens and anchor a at position n:
  d_1..d_{G-1} = drafter(anchor)
  the target runs once over [committed ; a, d_1..d_{G-1}] and yields
  y_j = argmax at position n+j (its choice for position n+j+1)
  verify -> tau = k+1; commit y_0..y_k
  the target's features at positions n..n+k (anchor + accepted drafts) are
  injected into the drafter; the next anchor is y_k.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .dflash import DraftModel, KVCache, inject, draft, verify, argmax_lowest
from .tiny_target import TinyTarget


class OracleDrafter:
    """The oracle's own drafter (inject + draft) for one sequence."""

    def __init__(self, model: DraftModel, cap: int):
        self.m = model
        self.kv = KVCache(model.cfg, 1, cap)

    def inject(self, feat_rows: np.ndarray) -> None:
        inject(self.m, self.kv, 0, feat_rows)

    def draft(self, anchor: int, gamma: int, history: List[int]) -> List[int]:
        return [int(t) for t in draft(self.m, self.kv, 0, anchor, gamma)]


class ConstantDrafter:
    """Always proposes the same token: accept length is 1 unless it happens to match."""

    def __init__(self, token: int = 0):
        self.token = token

    def inject(self, feat_rows) -> None:
        pass

    def draft(self, anchor, gamma, history):
        return [self.token] * (gamma - 1)


class CorruptedGreedyDrafter:
    """Proposes the target's own greedy continuation with seeded corruptions,
    so cycles see partial acceptances of every length."""

    def __init__(self, target: TinyTarget, seed: int = 0, p_corrupt: float = 0.25):
        self.t = target
        self.g = np.random.default_rng(seed)
        self.p = p_corrupt

    def inject(self, feat_rows) -> None:
        pass

    def draft(self, anchor, gamma, history):
        toks = list(history) + [anchor]
        out = []
        for _ in range(gamma - 1):
            logits, _ = self.t.forward(toks)
            nxt = int(argmax_lowest(logits[-1:])[0])
            if self.g.random() < self.p:
                nxt = (nxt + 1) % self.t.cfg.vocab
            out.append(nxt)
            toks.append(nxt)
        return out


def spec_decode(target: TinyTarget, drafter, prompt: List[int], n_tokens: int,
                gamma: int) -> Tuple[List[int], List[int]]:
    """Generate n_tokens with draft + verify cycles; returns (tokens, accept lengths)."""
    logits, hid = target.forward(prompt)
    drafter.inject(target.storage_features(hid))
    anchor = int(argmax_lowest(logits[-1:])[0])
    out = [anchor]
    seq = list(prompt)
    taus = []
    while len(out) < n_tokens:
        d = list(drafter.draft(anchor, gamma, seq))
        n = len(seq)
        logits, hid = target.forward(seq + [anchor] + d)
        y = argmax_lowest(logits[n: n + gamma])
        tau, committed, nxt = verify(d, y)
        feats = target.storage_features(hid)[n: n + tau]
        seq = seq + [anchor] + d[: tau - 1]
        drafter.inject(feats)
        out.extend(int(t) for t in committed[:tau])
        taus.append(tau)
        anchor = nxt
    return out[:n_tokens], taus
