"""The drafter's training objective: position-weighted block cross-entropy.

TEST INFRASTRUCTURE (see ``oracle/dflash.py``).  Source: "DFlash" technical
summary, §2.3 (training strategy), loss-weighting bullet: the cross-entropy of
the block's predictions is weighted so that early positions in the block count
more, because an early wrong token makes every later one useless; the weight of
block position k is w_k = exp(-(k - 1) / gamma).  The alignment bullet of the
same section says what the predictions are compared with: the outputs of the
frozen target model, i.e. the target's tokens at the block positions.

Readings where the pages are silent:
  * the predicted positions are the mask rows j = 1 .. gamma-1 of a block that
    starts at an anchor token (§2.3, random anchor sampling; the anchor itself is
    given, so it has no loss); block position k of the formula is j, so the
    first predicted token has weight 1;
  * the loss of a batch of blocks is the weighted mean
        L = sum_b sum_j w_j CE[b][j] / (B * sum_j w_j),
    a normalisation that leaves the direction of every gradient unchanged;
  * CE[b][j] = logsumexp(z[b][j]) - z[b][j][label] with the logits z of the
    drafter's forward pass exactly as drafting computes them (``draft``).

Parity unpinned: the normalisation of the batch loss and the mapping of block position k
to mask row j are readings; the weights, the cross-entropy and the gradient are pinned.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .dflash import DraftModel, KVCache, draft


def position_weights(gamma: int) -> np.ndarray:
    """w_j for the mask rows j = 1 .. gamma-1 (array index j-1): exp(-(j - 1) / gamma)."""
    j = np.arange(1, gamma, dtype=np.float64)
    return np.exp(-(j - 1.0) / gamma)


def cross_entropy_rows(z: np.ndarray, labels: Sequence[int]) -> np.ndarray:
    """CE of each row of logits z [rows][V] against labels [rows], in fp64:
    logsumexp(z) - z[label], the log-sum-exp taken around the row maximum."""
    z = np.asarray(z, dtype=np.float64)
    lab = np.asarray(labels, dtype=np.int64)
    mx = z.max(axis=-1)
    lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=-1))
    return lse - z[np.arange(z.shape[0]), lab]


def weighted_block_loss(ce: np.ndarray) -> float:
    """L = sum_b sum_j w_j CE[b][j] / (B * sum_j w_j) for CE [B][gamma-1]."""
    ce = np.asarray(ce, dtype=np.float64)
    w = position_weights(ce.shape[1] + 1)
    return float((ce * w[None, :]).sum() / (ce.shape[0] * w.sum()))


def block_loss(m: DraftModel, kv: KVCache, anchors: Sequence[int], labels: np.ndarray,
               gamma: int) -> Tuple[float, np.ndarray, np.ndarray]:
    """The objective over a batch of blocks: sequence b drafts from anchors[b] at its
    cached context, labels[b] [gamma-1] are the target's tokens at positions 1 ..
    gamma-1.  Returns (L, CE [B][gamma-1], logits [B][gamma-1][V])."""
    ces, zs = [], []
    for b, a in enumerate(anchors):
        _, _, z = draft(m, kv, b, int(a), gamma, return_all=True)
        ces.append(cross_entropy_rows(z, labels[b]))
        zs.append(z)
    ce = np.stack(ces)
    return weighted_block_loss(ce), ce, np.stack(zs)


def block_loss_grad(z: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """Gradient of ``weighted_block_loss(CE(z, labels))`` with respect to the logits
    z [B][gamma-1][V]: row (b, j) contributes w_j / (B * sum_j w_j) * CE[b][j], and the
    derivative of a row's cross-entropy is softmax(z[b][j]) minus the one-hot label."""
    z = np.asarray(z, dtype=np.float64)
    B, R, V = z.shape
    w = position_weights(R + 1)
    p = np.exp(z - z.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    onehot = np.zeros_like(p)
    lab = np.asarray(labels, dtype=np.int64)
    np.put_along_axis(onehot, lab[..., None], 1.0, axis=-1)
    return (w[None, :, None] / (B * w.sum())) * (p - onehot)
