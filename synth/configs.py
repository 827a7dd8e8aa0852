"""Workload shapes for one DFlash drafting + verification cycle.

The five shapes are drafters for targets named in "DFlash: Block Diffusion for
Flash Speculative Decoding" (gist.science summary, section 4, experiments:
Qwen3-4B/8B, Qwen3-Coder-30B, LLaMA-3.1-8B).  The drafter depth of 5 follows
section 3 (contribution 1) and the block of 16 tokens follows section 2.2
(parallel block diffusion).  The pages give no other hyper-parameter; every
other field is a stated reading (Qwen3 recipe: q/k RMSNorm, rotate-half RoPE,
no biases, eps 1e-6, theta 1e6).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str            # "f32" or "bf16": storage type of weights, K/V cache and features
    hidden: int           # H
    n_q: int              # query heads
    n_kv: int             # key/value heads (GQA groups of n_q // n_kv)
    head_dim: int         # D
    inter: int            # SwiGLU intermediate size I
    n_layers: int         # L draft layers
    n_feat: int           # F target layers whose hidden states are fused
    vocab: int            # V
    gamma: int            # block size (anchor + gamma-1 masks)
    ctx: int              # context length per sequence (fixed lengths)
    batch: int
    tied: bool = False    # LM head aliases the embedding table
    ctx_range: Optional[Tuple[int, int]] = None   # ragged lengths U{lo..hi} (inclusive)
    gammas: Optional[Tuple[int, ...]] = None      # dynamic block sizes, cycled per cycle
    plant_p: float = 0.845    # per-position agreement probability of planted targets
    rope_theta: float = 1.0e6
    eps: float = 1.0e-6
    index: int = 0            # seed stream index

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def mask_id(self) -> int:
        # The mask token is an ordinary embedding row: the last id of the vocabulary.
        return self.vocab - 1

    @property
    def gamma_max(self) -> int:
        return max(self.gammas) if self.gammas else self.gamma

    @property
    def max_ctx(self) -> int:
        return self.ctx_range[1] if self.ctx_range else self.ctx

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


C1 = Config("tiny_f32", "f32", hidden=256, n_q=4, n_kv=2, head_dim=64, inter=512,
            n_layers=2, n_feat=3, vocab=1024, gamma=8, ctx=64, batch=1,
            plant_p=0.8, index=1)
C2 = Config("qwen3_4b_drafter", "bf16", hidden=2560, n_q=32, n_kv=8, head_dim=128,
            inter=9728, n_layers=5, n_feat=5, vocab=151936, gamma=16, ctx=1024,
            batch=1, tied=True, index=2)
C3 = Config("qwen3_8b_drafter", "bf16", hidden=4096, n_q=32, n_kv=8, head_dim=128,
            inter=12288, n_layers=5, n_feat=5, vocab=151936, gamma=16, ctx=4096,
            batch=1, index=3)
C4 = Config("llama31_8b_drafter_b32", "bf16", hidden=4096, n_q=32, n_kv=8, head_dim=128,
            inter=14336, n_layers=5, n_feat=5, vocab=128256, gamma=16, ctx=4352,
            batch=32, ctx_range=(512, 8192), index=4)
C5 = Config("coder30b_drafter_longctx", "bf16", hidden=2048, n_q=32, n_kv=4, head_dim=128,
            inter=6144, n_layers=5, n_feat=5, vocab=151936, gamma=16, ctx=32768,
            batch=8, gammas=(16, 8), index=5)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}
ALIASES = {"C1": C1.name, "C2": C2.name, "C3": C3.name, "C4": C4.name, "C5": C5.name}


def get_config(name: str) -> Config:
    return CONFIGS[ALIASES.get(name, name)]


def tiny_config(**kw) -> Config:
    """A very small shape for brute-force checks; any field may be overridden."""
    base = Config("micro", "f32", hidden=32, n_q=4, n_kv=2, head_dim=8, inter=48,
                  n_layers=2, n_feat=2, vocab=16, gamma=4, ctx=5, batch=1,
                  plant_p=0.8, index=99)
    return base.with_(**kw)
