"""Seeded synthetic tensors for the drafting + verification cycle.

Every tensor is drawn from its own stream
``SeedSequence([20260205, cfg.index, crc32(name), block])`` so values do not
depend on generation order or thread count.  Large tensors are drawn in row
blocks on a thread pool (numpy's generators release the GIL).

Storage: bf16 configurations return ``uint16`` arrays holding bf16 bit patterns
(round-to-nearest-even of an fp32 draw); fp32 configurations return
``float32`` arrays.  Turning the bit patterns into numbers is left to each
consumer (the oracle widens them on the CPU, the GPU binding uploads them as
``torch.bfloat16``).

Distributions (the shapes and value ranges of the workloads in the pages'
experiments, which need trained weights and datasets that are not here):
  * every 2-D weight ``[rows][cols]`` ~ N(0, 1/cols) (fan-in scaling);
  * every 1-D norm scale ~ 1 + 0.1 N(0, 1) (not plain ones, so a kernel that
    drops a scale is caught);
  * target hidden states (features) ~ N(0, 1);
  * context K/V cache rows ~ N(0, 1) (after a per-head RMSNorm and RoPE,
    injected keys and values have unit RMS);
  * token ids uniform in [0, V).
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np

from .configs import Config

ROOT_SEED = 20260205
_BLOCK = 1 << 22          # values per independently seeded block
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _ss(cfg: Config, name: str, block: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence([ROOT_SEED, cfg.index, zlib.crc32(name.encode()), block])


def rng(cfg: Config, name: str, block: int = 0) -> np.random.Generator:
    return np.random.default_rng(_ss(cfg, name, block))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(cfg: Config, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """N(mean, std^2) draws in the config's storage format (bf16 bits or fp32)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    bf16 = cfg.dtype == "bf16"
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def fill(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        x = rng(cfg, name, b).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(x) if bf16 else x

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(min(_THREADS, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def tokens(cfg: Config, name: str, shape, lo: int = 0, hi: int = None) -> np.ndarray:
    hi = cfg.vocab if hi is None else hi
    return rng(cfg, name).integers(lo, hi, size=shape, dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------- weights

def layer_weight_shapes(cfg: Config) -> Dict[str, Tuple[int, ...]]:
    H, D, I = cfg.hidden, cfg.head_dim, cfg.inter
    return {
        "in_norm": (H,),
        "wq": (cfg.n_q * D, H),
        "wk": (cfg.n_kv * D, H),
        "wv": (cfg.n_kv * D, H),
        "q_norm": (D,),
        "k_norm": (D,),
        "wo": (H, cfg.n_q * D),
        "post_norm": (H,),
        "w_gate": (I, H),
        "w_up": (I, H),
        "w_down": (H, I),
    }


def global_weight_shapes(cfg: Config) -> Dict[str, Tuple[int, ...]]:
    H = cfg.hidden
    shapes = {
        "w_fuse": (H, cfg.n_feat * H),
        "embed": (cfg.vocab, H),
        "final_norm": (H,),
    }
    if not cfg.tied:
        shapes["lm_head"] = (cfg.vocab, H)
    return shapes


def _draw_weight(cfg: Config, name: str, shape) -> np.ndarray:
    if len(shape) == 1:
        return normal(cfg, name, shape, std=0.1, mean=1.0)
    return normal(cfg, name, shape, std=float(1.0 / np.sqrt(shape[1])))


def weights(cfg: Config, overrides: Dict[str, np.ndarray] = None) -> Dict[str, object]:
    """All drafter weights: {'w_fuse','embed','lm_head','final_norm','layers':[{...}]*L}.

    ``lm_head`` is the same array object as ``embed`` for tied configurations.
    ``overrides`` maps a global name or ``"layers.<l>.<name>"`` to a replacement.
    """
    overrides = overrides or {}
    W: Dict[str, object] = {}
    for name, shape in global_weight_shapes(cfg).items():
        W[name] = overrides.get(name, None)
        if W[name] is None:
            W[name] = _draw_weight(cfg, name, shape)
    if cfg.tied:
        W["lm_head"] = W["embed"]
    layers: List[Dict[str, np.ndarray]] = []
    for l in range(cfg.n_layers):
        lw = {}
        for name, shape in layer_weight_shapes(cfg).items():
            key = f"layers.{l}.{name}"
            lw[name] = overrides.get(key, None)
            if lw[name] is None:
                lw[name] = _draw_weight(cfg, key, shape)
        layers.append(lw)
    W["layers"] = layers
    return W


# --------------------------------------------------------------------------- per-cycle inputs

def context_lengths(cfg: Config) -> np.ndarray:
    if cfg.ctx_range is None:
        return np.full(cfg.batch, cfg.ctx, dtype=np.int32)
    lo, hi = cfg.ctx_range
    return rng(cfg, "ctx_len").integers(lo, hi + 1, size=cfg.batch).astype(np.int32)


def kv_capacity(cfg: Config, extra_rows: int = 0) -> int:
    """Cache rows per (layer, sequence, kv head): the longest context plus room for
    one block of gamma_max rows and ``extra_rows`` more, rounded up to 64."""
    need = cfg.max_ctx + cfg.gamma_max + extra_rows
    return (need + 63) // 64 * 64


def context_kv(cfg: Config, lengths: np.ndarray, cap: int, tag: str = "ctx") -> Tuple[np.ndarray, np.ndarray]:
    """Synthetic injected context: K and V caches ``[L][B][n_kv][cap][D]``.

    Rows ``>= lengths[b]`` are zero (they hold nothing yet).  Keys and values are
    drawn per (layer, sequence) so that a batch-1 slice equals the batch-B one.
    """
    L, B, nkv, D = cfg.n_layers, len(lengths), cfg.n_kv, cfg.head_dim
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    K = np.zeros((L, B, nkv, cap, D), dtype=dt)
    V = np.zeros((L, B, nkv, cap, D), dtype=dt)
    for l in range(L):
        for b in range(B):
            n = int(lengths[b])
            if n == 0:
                continue
            K[l, b, :, :n] = normal(cfg, f"{tag}.k.{l}.{b}", (nkv, n, D))
            V[l, b, :, :n] = normal(cfg, f"{tag}.v.{l}.{b}", (nkv, n, D))
    return K, V


def features(cfg: Config, batch: int, rows: int, tag: str = "feat") -> np.ndarray:
    """Target hidden states of the F tapped layers: ``[batch][rows][F][H]`` ~ N(0,1)."""
    return normal(cfg, tag, (batch, rows, cfg.n_feat, cfg.hidden))


def anchors(cfg: Config, batch: int, tag: str = "anchor") -> np.ndarray:
    return tokens(cfg, tag, (batch,))


def planted_accept(cfg: Config, shape, gamma: int, tag: str = "plant") -> np.ndarray:
    """Planted number of leading draft/target agreements k in [0, gamma-1].

    Each successive position agrees with probability ``cfg.plant_p``, so
    P(k >= j) = p**j truncated at gamma-1; the accept length is k + 1.
    """
    g = rng(cfg, tag)
    u = g.random(tuple(shape) + (gamma - 1,))
    agree = u < cfg.plant_p
    k = np.cumprod(agree, axis=-1).sum(axis=-1)
    return k.astype(np.int32)


def planted_targets(cfg: Config, draft: np.ndarray, k: np.ndarray, tag: str = "plant_y") -> np.ndarray:
    """Target argmax tokens y[b][gamma] that agree with ``draft`` for exactly k[b] positions.

    y_{j-1} = d_j for j <= k, y_k != d_{k+1} (when k < gamma-1), the rest uniform.
    ``draft`` is [B][gamma-1].  This builds an input; it does not verify anything.
    """
    B, gm1 = draft.shape
    g = rng(cfg, tag)
    y = g.integers(0, cfg.vocab, size=(B, gm1 + 1)).astype(np.int32)
    off = g.integers(1, cfg.vocab, size=B).astype(np.int64)
    for b in range(B):
        kb = int(k[b])
        y[b, :kb] = draft[b, :kb]
        if kb < gm1:
            y[b, kb] = (int(draft[b, kb]) + int(off[b])) % cfg.vocab
    return y

