"""Input-fusion conditioning: the alternative that DFlash's KV injection is measured against.

TEST INFRASTRUCTURE (see ``oracle/dflash.py``).  Source: "DFlash" technical
summary, §2.2, KV-injection bullet: methods that fuse the target's features only at
the input layer lose that information as the drafter gets deeper, whereas DFlash
feeds the fused context feature into every layer's key and value projections; §4
(ablations): KV injection beats input fusion for autoregressive and for block
drafters.  The pages give no formula for the input-fusion drafter; the plainest
reading that the rest supports, used here:

  * the fused context feature c_i = W_fuse rho(concat_f feat[i][f]) (the same
    fusion step as KV injection, ``fuse``) is the drafter's input hidden state at
    context position len + i, in place of a token embedding;
  * every draft layer runs over the new context rows with the drafter's own recipe
    (input RMSNorm, q/k per-head RMSNorm + RoPE, GQA attention, W_o, SwiGLU MLP);
    a context row attends to the cached context and to the new rows up to and
    including itself (context is history: causal);
  * each layer keeps the rows' rounded k and v at their positions in its own cache,
    so the block pass (``draft``) reads per-layer context K/V exactly as after KV
    injection; len advances by the number of rows.

Parity unpinned: that this is the pages' input-fusion drafter is a reading (they give no
formula); the computation itself is pinned (a torch causal-attention composite, layer 0
equal to KV injection, causality, chunking).

With one layer the two conditionings coincide (layer 0's K/V are the projections
of c in both); from the second layer on, input fusion's K/V come from hidden states
that passed through the layers below.
"""
from __future__ import annotations

import math

import numpy as np

from .dflash import DraftModel, KVCache, fuse, rms_norm, rope, silu, linear, softmax_rows


def inject_input_fusion(m: DraftModel, kv: KVCache, b: int, feat_rows: np.ndarray) -> np.ndarray:
    """Append the n feature rows of sequence b at positions len[b] .. len[b]+n-1 by running
    every draft layer over their fused features; returns the final hidden rows [n][H]."""
    cfg = m.cfg
    rho = m.num.rho
    D, nq, nkv = cfg.head_dim, cfg.n_q, cfg.n_kv
    g = nq // nkv
    if feat_rows.shape[0] == 0:
        return np.zeros((0, cfg.hidden))
    x = fuse(m, feat_rows)                                   # [n][H]
    n = x.shape[0]
    C = int(kv.len[b])
    pos = np.arange(C, C + n)
    # row i sees keys 0 .. C + i
    allowed = np.arange(C + n)[None, :] <= (C + np.arange(n))[:, None]
    for l, lw in enumerate(m.layers):
        a = rho(rms_norm(x, lw["in_norm"], cfg.eps))
        q = linear(a, lw["wq"]).reshape(n, nq, D)
        k = linear(a, lw["wk"]).reshape(n, nkv, D)
        v = linear(a, lw["wv"]).reshape(n, nkv, D)
        q = rho(rope(rms_norm(q, lw["q_norm"], cfg.eps), pos, cfg.rope_theta))
        k = rho(rope(rms_norm(k, lw["k_norm"], cfg.eps), pos, cfg.rope_theta))
        v = rho(v)
        kv.k[l, b, :, C:C + n, :] = k.transpose(1, 0, 2)
        kv.v[l, b, :, C:C + n, :] = v.transpose(1, 0, 2)
        o = np.empty((n, nq, D))
        for h in range(nq):
            keys = kv.k[l, b, h // g, :C + n]
            vals = kv.v[l, b, h // g, :C + n]
            s = (q[:, h] @ keys.T) / math.sqrt(D)
            o[:, h] = softmax_rows(np.where(allowed, s, -np.inf)) @ vals
        x = x + linear(rho(o.reshape(n, nq * D)), lw["wo"])
        a2 = rho(rms_norm(x, lw["post_norm"], cfg.eps))
        x = x + linear(rho(silu(linear(a2, lw["w_gate"])) * linear(a2, lw["w_up"])), lw["w_down"])
    kv.len[b] = C + n
    return x
