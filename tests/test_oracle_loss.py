"""Pins for the oracle's position-weighted block cross-entropy (the drafter's
training objective, "DFlash" technical summary section 2.3, loss weighting)."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from synth import gen
from oracle import dflash as O
from oracle import loss as OL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "loss_weights.json")


def test_weights_match_hand_evaluated_formula():
    g = json.load(open(GOLDEN))
    w = OL.position_weights(g["gamma"])
    assert w.shape == (g["gamma"] - 1,)
    np.testing.assert_allclose(w, g["weights"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("gamma", [2, 8, 16])
def test_weights_start_at_one_and_decay(gamma):
    w = OL.position_weights(gamma)
    assert w.shape == (gamma - 1,)
    assert w[0] == 1.0                                  # the first predicted position has weight 1
    assert np.all(np.diff(w) < 0)                       # early positions count more
    assert np.all(w > math.exp(-1.0))                   # (k - 1) / gamma < 1 for every mask row


def test_cross_entropy_equals_torch_library_routine():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(7, 301)) * 3.0
    lab = rng.integers(0, 301, size=7)
    ref = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(lab), reduction="none").numpy()
    np.testing.assert_allclose(OL.cross_entropy_rows(z, lab), ref, rtol=1e-13, atol=1e-13)


def test_cross_entropy_closed_forms():
    V = 1000
    z = np.zeros((3, V))
    np.testing.assert_allclose(OL.cross_entropy_rows(z, [0, 5, 999]), math.log(V), rtol=1e-14)
    # shift invariance and no overflow at large logits
    rng = np.random.default_rng(2)
    z = rng.normal(size=(4, 50))
    lab = [1, 2, 3, 4]
    np.testing.assert_allclose(OL.cross_entropy_rows(z + 1e4, lab), OL.cross_entropy_rows(z, lab), rtol=1e-9)
    # a dominant label logit gives ~0, a label far below the rest gives its gap
    z = np.zeros((1, 10))
    z[0, 3] = 50.0
    assert OL.cross_entropy_rows(z, [3])[0] < 1e-20
    np.testing.assert_allclose(OL.cross_entropy_rows(z, [4])[0], 50.0, rtol=1e-12)


def test_weighted_mean_golden_example_and_properties():
    g = json.load(open(GOLDEN))
    ex = g["example"]
    assert OL.weighted_block_loss(np.array(ex["ce"])) == pytest.approx(ex["loss"], rel=1e-14)
    rng = np.random.default_rng(3)
    ce = rng.uniform(0, 10, size=(5, 15))
    # a constant CE is returned unchanged (weights are normalised)
    assert OL.weighted_block_loss(np.full((5, 15), 2.5)) == pytest.approx(2.5, rel=1e-14)
    # order of the blocks in the batch does not matter; the loss is linear in CE
    assert OL.weighted_block_loss(ce[::-1]) == pytest.approx(OL.weighted_block_loss(ce), rel=1e-14)
    assert OL.weighted_block_loss(3 * ce) == pytest.approx(3 * OL.weighted_block_loss(ce), rel=1e-14)
    # between the smallest and the largest row loss
    L = OL.weighted_block_loss(ce)
    assert ce.min() <= L <= ce.max()
    # a later position moves the loss less than an earlier one
    a = np.zeros((1, 15)); a[0, 0] = 1.0
    b = np.zeros((1, 15)); b[0, 14] = 1.0
    assert OL.weighted_block_loss(a) > OL.weighted_block_loss(b)


def test_block_loss_uses_the_draft_forward_logits():
    cfg = synth.tiny_config(gamma=8)
    m = O.DraftModel(cfg, gen.weights(cfg))
    kv = O.KVCache(cfg, 2, 64)
    for b, n in enumerate([5, 0]):
        if n:
            O.inject(m, kv, b, O.decode_storage(gen.features(cfg, 1, n, tag=f"loss.f{b}"))[0])
    anchors = [7, 11]
    d0, _, z0 = O.draft(m, kv, 0, anchors[0], 8, return_all=True)
    d1, _, z1 = O.draft(m, kv, 1, anchors[1], 8, return_all=True)
    # labels = the drafter's own argmax tokens: every CE is in [0, log V]
    L, ce, z = OL.block_loss(m, kv, anchors, np.stack([d0, d1]), 8)
    np.testing.assert_array_equal(z[0], z0)
    np.testing.assert_array_equal(z[1], z1)
    assert np.all(ce >= 0) and np.all(ce <= math.log(cfg.vocab) + 1e-12)
    # labels = each row's least likely token: CE >= log V
    worst = np.stack([np.argmin(z0, axis=-1), np.argmin(z1, axis=-1)])
    _, ce_w, _ = OL.block_loss(m, kv, anchors, worst, 8)
    assert np.all(ce_w >= math.log(cfg.vocab))
    assert L == pytest.approx(OL.weighted_block_loss(ce), rel=1e-15)


def test_gradient_equals_torch_autograd():
    """d L / d logits against torch autograd through F.cross_entropy (library routines)."""
    rng = np.random.default_rng(4)
    B, R, V = 3, 7, 50
    z = rng.normal(size=(B, R, V)) * 2.0
    lab = rng.integers(0, V, size=(B, R))
    zt = torch.tensor(z, requires_grad=True)
    ce = F.cross_entropy(zt.reshape(-1, V), torch.from_numpy(lab).reshape(-1), reduction="none").reshape(B, R)
    w = torch.from_numpy(OL.position_weights(R + 1))
    L = (ce * w[None, :]).sum() / (B * w.sum())
    L.backward()
    g = OL.block_loss_grad(z, lab)
    np.testing.assert_allclose(g, zt.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert L.item() == pytest.approx(OL.weighted_block_loss(OL.cross_entropy_rows(z.reshape(-1, V), lab.reshape(-1)).reshape(B, R)), rel=1e-13)
    # every row's gradient sums to zero (softmax minus one-hot)
    np.testing.assert_allclose(g.sum(axis=-1), 0.0, atol=1e-15)
