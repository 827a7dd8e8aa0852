"""Plain CPU oracle for one DFlash drafting + verification cycle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``.  The GPU library never calls it, and it shares no code with the
GPU path: the only thing both sides import is the seeded input generator
(``synth``), which performs none of the method's arithmetic.

What is computed, and where the pages say so
--------------------------------------------
Sources: "DFlash: Block Diffusion for Flash Speculative Decoding" — the
gist.science technical summary (Japanese and Dutch pages, same sections) and
the abstract on the fugumt.com paper page.

* Context features (summary §2.2, first bullet): hidden states of a fixed set
  of target layers, spread from shallow to deep, are concatenated and projected
  to one compact context feature.                                -> ``fuse``
* KV injection (summary §2.2, second bullet; §3 item 2): the context feature
  is persistent information fed into the key and value projections of every
  draft layer and stored in that layer's draft KV cache.          -> ``inject``
* Parallel block diffusion (summary §2.2, third bullet; abstract): one forward
  pass predicts a whole block of masked tokens (e.g. 16).         -> ``draft``
* The block starts at a clean anchor token produced by the target (summary
  §2.3, random anchor sampling, which mirrors inference).
* The drafter shares the target's frozen token embedding and LM head (summary
  §2.3, architecture bullet).
* Lossless greedy verification: the target checks the drafts in parallel and
  the output equals greedy decoding (summary §1, §4 speed-ups vs. greedy, §5;
  abstract).  Acceptance length counts tokens per cycle (summary §4).
                                                                  -> ``verify``

Readings where the pages are silent (each one is listed with its reason in the
design notes of this repository):
  R3  no norm after W_fuse; context rows pass through each layer's own input
      RMSNorm before W_k / W_v (``shared_fuse_norm`` switches to one shared
      RMSNorm after fusion instead).
  R4  Qwen3 recipe: input RMSNorm, per-head q/k RMSNorm over D, then RoPE;
      V has no per-head norm; no biases.
  R5  rotate-half RoPE, theta from the config, absolute positions
      (context 0..C-1, block C..C+gamma-1); angles evaluated here in fp64.
  R6  the mask token is an ordinary embedding row (id V-1).
  R7  only mask rows 1..gamma-1 go through the LM head; row j predicts the
      token at position C+j.
  R8  no causal mask inside the block, full context visible, scale 1/sqrt(D),
      q head h reads kv head h // (n_q/n_kv).
  R9  one final RMSNorm before the LM head.
  R10 eps = 1e-6.
  R11 argmax ties go to the lowest index.
  R12 accept length = accepted drafts + 1 bonus token.
  R14 the block's own K/V are not kept in the cache.

Parity unpinned: R3-R7, R9, R10 and the weight initialisation are conventions the
pages do not fix.  The functions that implement them are pinned (library routines,
closed forms, brute force), but which convention is the pages' one is not: an
independent oracle choosing differently would disagree there.

Precision contract: numbers are carried in ``dtype`` (fp64 by default).  For
bf16 configurations ``rho`` rounds to the nearest bf16 (ties to even) exactly
at the points the GPU path must also round: every GEMM input (A operand), the
q/k/v vectors, and the K/V rows stored in the cache.  For fp32 configurations
``rho`` is the identity.  The residual stream, norms, RoPE, softmax and all
sums stay in ``dtype``.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------- scalars

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits), ties to even.

    Written from the definition of the format: a finite x = m * 2**e with
    0.5 <= |m| < 1 keeps 8 significant bits of m.  Valid for the normal range
    (|x| >= 2**-126), which is all this oracle ever sees.
    """
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def decode_storage(a: np.ndarray, dtype=F64) -> np.ndarray:
    """Storage array (bf16 bit patterns as uint16, or fp32) -> numbers in ``dtype``."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)
    return a.astype(dtype)


class Numerics:
    """Where and how the oracle rounds (see the module docstring)."""

    def __init__(self, storage: str, dtype=F64):
        self.storage = storage
        self.dtype = dtype

    def rho(self, x: np.ndarray) -> np.ndarray:
        if self.storage == "bf16":
            return round_bf16(x).astype(self.dtype)
        return np.asarray(x, dtype=self.dtype)


# ----------------------------------------------------------------------------- primitives

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Angle of pair i at position p: p * theta**(-2i/D); shape [len(pos)][D/2]."""
    i = np.arange(head_dim // 2, dtype=F64)
    inv = theta ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=F64)[:, None] * inv[None, :]


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE.  x: [..., P, H, D] with positions pos[P] on axis -3.

    Pair (x_i, x_{i+D/2}) is rotated by the angle of pair i.
    """
    D = x.shape[-1]
    ang = rope_angles(pos, D, theta)              # [P][D/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def linear(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = a W^T for a weight stored [out][in] (one library matmul)."""
    return a @ w.T


def softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def block_attention(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
                    k_blk: np.ndarray, v_blk: np.ndarray) -> np.ndarray:
    """GQA attention of block queries over [context ; block] keys, no mask.

    q      [G][n_q][D]   block queries (G = gamma)
    k_ctx  [n_kv][C][D]  injected context keys (C may be 0)
    k_blk  [G][n_kv][D]  the block's own keys
    Query head h reads kv head h // (n_q / n_kv).  Returns [G][n_q][D].
    """
    G, n_q, D = q.shape
    n_kv = k_blk.shape[1]
    g = n_q // n_kv
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    for h in range(n_q):
        hk = h // g
        keys = np.concatenate([k_ctx[hk], k_blk[:, hk, :]], axis=0)
        vals = np.concatenate([v_ctx[hk], v_blk[:, hk, :]], axis=0)
        p = softmax_rows((q[:, h, :] @ keys.T) * scale)
        out[:, h, :] = p @ vals
    return out


def argmax_lowest(z: np.ndarray) -> np.ndarray:
    """Row-wise argmax; among equal maxima the lowest index wins (R11)."""
    return np.argmax(z, axis=-1).astype(np.int32)


# ----------------------------------------------------------------------------- model state

class DraftModel:
    """Drafter weights decoded from storage, plus the configuration."""

    def __init__(self, cfg, W: Dict[str, object], dtype=F64):
        self.cfg = cfg
        self.num = Numerics(cfg.dtype, dtype)
        dec = lambda a: decode_storage(a, dtype)
        self.w_fuse = dec(W["w_fuse"])
        self.embed = dec(W["embed"])
        self.lm_head = self.embed if W["lm_head"] is W["embed"] else dec(W["lm_head"])
        self.final_norm = dec(W["final_norm"])
        self.layers = [{k: dec(v) for k, v in lw.items()} for lw in W["layers"]]


class KVCache:
    """Draft KV cache: K, V [L][B][n_kv][cap][D] and lengths len[B]."""

    def __init__(self, cfg, batch: int, cap: int, dtype=F64):
        L, nkv, D = cfg.n_layers, cfg.n_kv, cfg.head_dim
        self.k = np.zeros((L, batch, nkv, cap, D), dtype=dtype)
        self.v = np.zeros((L, batch, nkv, cap, D), dtype=dtype)
        self.len = np.zeros(batch, dtype=np.int64)
        self.cap = cap

    @classmethod
    def from_storage(cls, cfg, K: np.ndarray, V: np.ndarray, lengths, dtype=F64) -> "KVCache":
        kv = cls(cfg, K.shape[1], K.shape[3], dtype)
        kv.k[...] = decode_storage(K, dtype)
        kv.v[...] = decode_storage(V, dtype)
        kv.len[:] = np.asarray(lengths, dtype=np.int64)
        return kv


# ----------------------------------------------------------------------------- stage 1+2: inject

def fuse(m: DraftModel, feat_rows: np.ndarray) -> np.ndarray:
    """Stage 1: concatenate the F tapped layers (shallow -> deep) and project.

    feat_rows [n][F][H] (decoded) -> c [n][H];  c = W_fuse rho(u).
    """
    n = feat_rows.shape[0]
    u = feat_rows.reshape(n, -1)                       # [n][F*H], ascending depth
    return linear(m.num.rho(u), m.w_fuse)


def context_kv_rows(m: DraftModel, c: np.ndarray, pos: np.ndarray,
                    shared_fuse_norm: Optional[np.ndarray] = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Stage 2 per layer: the fused feature through that layer's K/V projections.

    Returns [(k, v)] per layer with k, v of shape [n][n_kv][D], already rho'd.
    """
    cfg = m.cfg
    n = c.shape[0]
    if shared_fuse_norm is not None:
        c = rms_norm(c, shared_fuse_norm, cfg.eps)
    out = []
    for lw in m.layers:
        ch = m.num.rho(rms_norm(c, lw["in_norm"], cfg.eps))
        k = linear(ch, lw["wk"]).reshape(n, cfg.n_kv, cfg.head_dim)
        v = linear(ch, lw["wv"]).reshape(n, cfg.n_kv, cfg.head_dim)
        k = rope(rms_norm(k, lw["k_norm"], cfg.eps), pos, cfg.rope_theta)
        out.append((m.num.rho(k), m.num.rho(v)))
    return out


def inject(m: DraftModel, kv: KVCache, b: int, feat_rows: np.ndarray,
           shared_fuse_norm: Optional[np.ndarray] = None) -> None:
    """Append the n feature rows of sequence b at positions len[b] .. len[b]+n-1."""
    n = feat_rows.shape[0]
    if n == 0:
        return
    C = int(kv.len[b])
    if C + n > kv.cap:
        raise ValueError("KV capacity exceeded")
    pos = np.arange(C, C + n)
    c = fuse(m, feat_rows)
    for l, (k, v) in enumerate(context_kv_rows(m, c, pos, shared_fuse_norm)):
        kv.k[l, b, :, C:C + n, :] = k.transpose(1, 0, 2)
        kv.v[l, b, :, C:C + n, :] = v.transpose(1, 0, 2)
    kv.len[b] = C + n


# ----------------------------------------------------------------------------- stage 3: draft

def draft(m: DraftModel, kv: KVCache, b: int, anchor: int, gamma: int,
          return_all: bool = False):
    """Stage 3: one forward pass over [anchor, MASK x (gamma-1)] for sequence b.

    Returns the gamma-1 draft tokens (and, with ``return_all``, the final
    residual stream x [gamma][H] and the logits [gamma-1][V]).
    """
    cfg = m.cfg
    rho = m.num.rho
    C = int(kv.len[b])
    D, nq, nkv = cfg.head_dim, cfg.n_q, cfg.n_kv
    ids = np.array([anchor] + [cfg.mask_id] * (gamma - 1), dtype=np.int64)
    pos = np.arange(C, C + gamma)
    x = m.embed[ids].copy()                                     # [G][H]
    for l, lw in enumerate(m.layers):
        a = rho(rms_norm(x, lw["in_norm"], cfg.eps))
        q = linear(a, lw["wq"]).reshape(gamma, nq, D)
        k = linear(a, lw["wk"]).reshape(gamma, nkv, D)
        v = linear(a, lw["wv"]).reshape(gamma, nkv, D)
        q = rho(rope(rms_norm(q, lw["q_norm"], cfg.eps), pos, cfg.rope_theta))
        k = rho(rope(rms_norm(k, lw["k_norm"], cfg.eps), pos, cfg.rope_theta))
        v = rho(v)
        o = block_attention(q, kv.k[l, b, :, :C, :], kv.v[l, b, :, :C, :], k, v)
        x = x + linear(rho(o.reshape(gamma, nq * D)), lw["wo"])
        a2 = rho(rms_norm(x, lw["post_norm"], cfg.eps))
        hmid = silu(linear(a2, lw["w_gate"])) * linear(a2, lw["w_up"])
        x = x + linear(rho(hmid), lw["w_down"])
    z = linear(rho(rms_norm(x[1:], m.final_norm, cfg.eps)), m.lm_head)   # mask rows only
    d = argmax_lowest(z)
    if return_all:
        return d, x, z
    return d


# ----------------------------------------------------------------------------- stage 4: verify

def verify(draft_tokens: Sequence[int], target_tokens: Sequence[int]) -> Tuple[int, np.ndarray, int]:
    """Greedy verification of one block.

    draft_tokens  d_1 .. d_{G-1}   (array index j-1 holds d_j)
    target_tokens y_0 .. y_{G-1}   (the target's argmax at the block positions;
                                    y_{j-1} is its choice for the position d_j fills)
    k = number of leading j with d_j == y_{j-1}; tau = k + 1 (the bonus token);
    committed = y_0 .. y_k; next anchor = y_k.
    Returns (tau, committed[G] padded with -1, next_anchor).
    """
    d = list(draft_tokens)
    y = list(target_tokens)
    G = len(y)
    assert len(d) == G - 1
    k = 0
    while k < G - 1 and d[k] == y[k]:
        k += 1
    committed = np.full(G, -1, dtype=np.int32)
    committed[: k + 1] = y[: k + 1]
    return k + 1, committed, int(y[k])


# ----------------------------------------------------------------------------- whole cycle

def cycle(m: DraftModel, kv: KVCache, feat: np.ndarray, n_new: Sequence[int],
          anchors: Sequence[int], gamma: int, target_fn) -> Dict[str, np.ndarray]:
    """inject -> draft -> verify for every sequence of the batch.

    feat [B][rows][F][H] decoded; ``target_fn(b, drafts) -> y[gamma]`` stands in
    for the target's parallel verification forward.
    """
    B = len(anchors)
    out = {"draft": np.zeros((B, gamma - 1), np.int32), "accept_len": np.zeros(B, np.int32),
           "committed": np.zeros((B, gamma), np.int32), "next_anchor": np.zeros(B, np.int32)}
    for b in range(B):
        inject(m, kv, b, feat[b, : int(n_new[b])])
        d = draft(m, kv, b, int(anchors[b]), gamma)
        tau, com, nxt = verify(d, target_fn(b, d))
        out["draft"][b] = d
        out["accept_len"][b] = tau
        out["committed"][b] = com
        out["next_anchor"][b] = nxt
    return out
