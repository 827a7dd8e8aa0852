"""A tiny random-init causal target model for the losslessness check.

TEST INFRASTRUCTURE (see ``oracle/dflash.py``).  The target follows the same
recipe as the drafter (RMSNorm, q/k RMSNorm + rotate-half RoPE, GQA, SwiGLU)
but with a causal mask, and it shares the drafter's token embedding and LM
head ("DFlash" technical summary, §2.3 architecture bullet: the drafter reuses
the target's frozen embedding and LM head).  Its hidden states at F layers
spread uniformly from shallow to deep are the context features (summary
§2.2, context-feature extraction).  Layer taps: decoder layers
round(linspace(1, N_t, F)) (1-based outputs, before the final norm).

Everything is fp64 with no rounding: the target only has to be a fixed,
deterministic greedy decoder.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from synth import gen
from .dflash import (decode_storage, rms_norm, rope, silu, linear, softmax_rows,
                     argmax_lowest, round_bf16)


class TinyTarget:
    def __init__(self, cfg, draft_model, n_layers: int = 4):
        self.cfg = cfg
        self.n_layers = n_layers
        tcfg = cfg.with_(n_layers=n_layers)
        W = gen.weights(tcfg.with_(index=cfg.index + 1000))
        dec = lambda a: decode_storage(a, np.float64)
        self.layers = [{k: dec(v) for k, v in lw.items()} for lw in W["layers"]]
        self.final_norm = dec(W["final_norm"])
        self.embed = draft_model.embed
        self.lm_head = draft_model.lm_head
        F = cfg.n_feat
        self.taps = [int(round(t)) for t in np.linspace(1, n_layers, F)]

    def forward(self, tokens: List[int]) -> Tuple[np.ndarray, List[np.ndarray]]:
        """Causal forward over the whole sequence; returns logits [n][V] and the
        residual stream after every decoder layer (index i = after layer i+1)."""
        cfg = self.cfg
        n = len(tokens)
        D, nq, nkv = cfg.head_dim, cfg.n_q, cfg.n_kv
        g = nq // nkv
        pos = np.arange(n)
        x = self.embed[np.asarray(tokens, dtype=np.int64)].copy()
        causal = np.tril(np.ones((n, n), dtype=bool))
        hiddens = []
        for lw in self.layers:
            a = rms_norm(x, lw["in_norm"], cfg.eps)
            q = rope(rms_norm(linear(a, lw["wq"]).reshape(n, nq, D), lw["q_norm"], cfg.eps), pos, cfg.rope_theta)
            k = rope(rms_norm(linear(a, lw["wk"]).reshape(n, nkv, D), lw["k_norm"], cfg.eps), pos, cfg.rope_theta)
            v = linear(a, lw["wv"]).reshape(n, nkv, D)
            o = np.empty((n, nq, D))
            for h in range(nq):
                s = (q[:, h] @ k[:, h // g].T) / math.sqrt(D)
                s = np.where(causal, s, -np.inf)
                o[:, h] = softmax_rows(s) @ v[:, h // g]
            x = x + linear(o.reshape(n, nq * D), lw["wo"])
            a2 = rms_norm(x, lw["post_norm"], cfg.eps)
            x = x + linear(silu(linear(a2, lw["w_gate"])) * linear(a2, lw["w_up"]), lw["w_down"])
            hiddens.append(x.copy())
        logits = linear(rms_norm(x, self.final_norm, cfg.eps), self.lm_head)
        return logits, hiddens

    def features(self, hiddens: List[np.ndarray]) -> np.ndarray:
        """[n][F][H]: the tapped layers' hidden states, shallow to deep."""
        return np.stack([hiddens[t - 1] for t in self.taps], axis=1)

    def storage_features(self, hiddens: List[np.ndarray]) -> np.ndarray:
        """Features as the drafter receives them: bf16-exact values for bf16 configs."""
        f = self.features(hiddens)
        return round_bf16(f) if self.cfg.dtype == "bf16" else f.astype(np.float32).astype(np.float64)


def greedy(target: TinyTarget, prompt: List[int], n_tokens: int) -> List[int]:
    """Plain greedy autoregressive decoding: n_tokens new tokens."""
    toks = list(prompt)
    for _ in range(n_tokens):
        logits, _ = target.forward(toks)
        toks.append(int(argmax_lowest(logits[-1:])[0]))
    return toks[len(prompt):]
