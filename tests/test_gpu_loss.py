"""GPU parity of the drafter's training objective (position-weighted block
cross-entropy, "DFlash" technical summary section 2.3) against the oracle: the
weight-streaming LM head at few rows, the tiled one at 128 rows with a vocabulary
whose last tile is partial, a bad label, and determinism."""
import math

import numpy as np
import pytest

import synth
from synth import gen
from oracle import loss as OL

from gpu_support import Pair, log, rel_err, tol

pytestmark = pytest.mark.gpu

# 128 block rows (batch 8 x gamma 16) and V = 40000: 313 LM-head blocks of 128 rows
# (the last one half full), enough for the tiled GEMM
BIGV = synth.Config("loss_bigv_bf16", "bf16", hidden=256, n_q=4, n_kv=2, head_dim=128, inter=512,
                    n_layers=1, n_feat=2, vocab=40000, gamma=16, ctx=200, batch=8, index=84)
MINI = synth.Config("loss_mini_bf16", "bf16", hidden=256, n_q=4, n_kv=2, head_dim=128, inter=512,
                    n_layers=2, n_feat=2, vocab=1000, gamma=16, ctx=300, batch=3, index=85)


def _labels(P, anchors, gamma, tag):
    """Half of the rows labelled with the oracle drafter's own choice, half at random."""
    cfg, B = P.cfg, P.batch
    d, _, _ = P.oracle_draft(anchors, gamma)
    rnd = gen.tokens(cfg, f"{tag}.labels", (B, gamma - 1))
    pick = gen.rng(cfg, f"{tag}.pick").random((B, gamma - 1)) < 0.5
    return np.where(pick, d, rnd).astype(np.int32)


def _loss_case(cfg, batch, lengths, gamma, tag):
    import torch
    cap = gen.kv_capacity(cfg, 64)
    log(f"case {cfg.name} batch={batch} lengths={list(lengths)} gamma={gamma} cap={cap}")
    P = Pair(cfg, batch, cap, 16)
    P.set_context(lengths, tag=tag)
    anchors = gen.tokens(cfg, f"{tag}.anchor", (batch,))
    labels = _labels(P, anchors, gamma, tag)
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    row = torch.full((batch, gamma - 1), float("nan"), dtype=torch.float32, device="cuda")
    lg = torch.full((batch, gamma - 1, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    P.dfl.block_loss(P.model, P.cache, gamma, P.dev_i32(anchors), P.dev_i32(labels), loss, P.ws, row, lg)
    torch.cuda.synchronize()
    L_ref, ce_ref, z_ref = OL.block_loss(P.om, P.okv, anchors, labels, gamma)
    got_L, got_ce, got_z = float(loss.item()), row.cpu().numpy(), lg.cpu().numpy()
    e_z, e_ce = rel_err(got_z, z_ref), rel_err(got_ce, ce_ref)
    e_L = abs(got_L - L_ref) / abs(L_ref)
    log(f"  loss gpu={got_L:.6f} oracle={L_ref:.6f} rel={e_L:.2e}; row CE rel={e_ce:.2e}; logits rel={e_z:.2e}")
    assert P.status() == 0
    assert np.isfinite(got_ce).all()
    assert e_z < tol(cfg) and e_ce < tol(cfg) and e_L < tol(cfg)
    # the device's own reduction of its row losses, in fp64, agrees closely
    assert abs(got_L - OL.weighted_block_loss(got_ce)) <= 1e-5 * abs(got_L)
    # determinism: a second call gives the same bits; with the gradient, written in place
    # over the logits (no dbg_logits) and next to separate logits, both against the oracle
    loss2 = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    g_in = torch.full((batch, gamma - 1, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    P.dfl.block_loss(P.model, P.cache, gamma, P.dev_i32(anchors), P.dev_i32(labels), loss2, P.ws, dlogits=g_in)
    lg2 = torch.full_like(g_in, float("nan"))
    g_sep = torch.full_like(g_in, float("nan"))
    P.dfl.block_loss(P.model, P.cache, gamma, P.dev_i32(anchors), P.dev_i32(labels), loss2, P.ws,
                     dbg_logits=lg2, dlogits=g_sep)
    torch.cuda.synchronize()
    assert float(loss2.item()) == got_L
    g_ref = OL.block_loss_grad(z_ref, labels)
    g_in, g_sep = g_in.cpu().numpy(), g_sep.cpu().numpy()
    e_g = rel_err(g_in, g_ref)
    log(f"  dlogits rel={e_g:.2e}")
    assert np.isfinite(g_in).all() and e_g < tol(cfg)
    np.testing.assert_array_equal(g_in, g_sep)
    np.testing.assert_array_equal(lg2.cpu().numpy(), got_z)
    # softmax minus one-hot: every row's gradient sums to ~0
    assert np.abs(g_in.astype(np.float64).sum(axis=-1)).max() < 1e-5
    return P, anchors, labels


def test_block_loss_fp32_tiny():
    cfg = synth.get_config("C1")
    _loss_case(cfg, 1, [cfg.ctx], cfg.gamma, "loss.c1")


def test_block_loss_bf16_ragged_batch():
    _loss_case(MINI, 3, [0, 300, 17], 16, "loss.mini")
    _loss_case(MINI, 3, [5, 0, 299], 5, "loss.mini5")


def test_block_loss_tiled_lm_head_partial_last_tile():
    _loss_case(BIGV, 8, [200, 0, 1, 64, 199, 100, 150, 2], 16, "loss.bigv")


def test_block_loss_bad_label_sets_status_and_nan():
    import torch
    P, anchors, labels = _loss_case(MINI, 3, [10, 20, 30], 8, "loss.bad")
    labels = labels.copy()
    labels[1, 3] = MINI.vocab            # out of range
    loss = torch.zeros((1,), dtype=torch.float32, device="cuda")
    row = torch.zeros((3, 7), dtype=torch.float32, device="cuda")
    P.dfl.block_loss(P.model, P.cache, 8, P.dev_i32(anchors), P.dev_i32(labels), loss, P.ws, row)
    torch.cuda.synchronize()
    r = row.cpu().numpy()
    assert P.status() & P.dfl._abi.STATUS_BAD_TOKEN
    assert math.isnan(float(loss.item())) and math.isnan(r[1, 3])
    assert np.isfinite(np.delete(r.ravel(), 1 * 7 + 3)).all()


def test_block_loss_on_randomly_anchored_blocks_of_a_target_decode():
    """The training objective as the summary's section 2.3 sets it up: a frozen (tiny,
    random-init) target decodes a response; anchors are drawn uniformly from the response;
    each block's context is the target's tapped hidden states before its anchor (injected),
    its labels the target's own tokens after the anchor.  GPU loss, row losses and gradient
    against the oracle on the same blocks."""
    import torch
    from oracle.tiny_target import TinyTarget, greedy
    cfg = synth.get_config("C1")
    B, G = 3, cfg.gamma
    cap = gen.kv_capacity(cfg, 64)
    P = Pair(cfg, B, cap, 64)
    tt = TinyTarget(cfg, P.om)
    prompt = [int(t) for t in gen.tokens(cfg, "loss.anchors.prompt", (9,))]
    seq = prompt + greedy(tt, prompt, 40)
    _, hiddens = tt.forward(seq)
    feats = tt.storage_features(hiddens)                          # [n][F][H], what injection reads
    rng = gen.rng(cfg, "loss.anchors.draw")
    anchors_pos = [int(a) for a in rng.integers(len(prompt), len(seq) - G + 1, size=B)]
    log(f"case random anchors at {anchors_pos} of a {len(seq)}-token sequence")
    rows = max(anchors_pos)
    feat = np.zeros((B, rows) + feats.shape[1:], dtype=np.float64)
    for b, a in enumerate(anchors_pos):
        feat[b, :a] = feats[:a]
    P.inject(feat.astype(np.float32), np.array(anchors_pos, dtype=np.int32))
    torch.cuda.synchronize()
    assert P.status() == 0 and list(P.cache.len.cpu().numpy()[:B]) == anchors_pos
    anchors = np.array([seq[a] for a in anchors_pos], dtype=np.int32)
    labels = np.array([seq[a + 1:a + G] for a in anchors_pos], dtype=np.int32)
    loss = torch.zeros((1,), dtype=torch.float32, device="cuda")
    row = torch.zeros((B, G - 1), dtype=torch.float32, device="cuda")
    dz = torch.zeros((B, G - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    P.dfl.block_loss(P.model, P.cache, G, P.dev_i32(anchors), P.dev_i32(labels), loss, P.ws, row, dlogits=dz)
    torch.cuda.synchronize()
    L_ref, ce_ref, z_ref = OL.block_loss(P.om, P.okv, anchors, labels, G)
    e_L = abs(float(loss.item()) - L_ref) / abs(L_ref)
    e_ce = rel_err(row.cpu().numpy(), ce_ref)
    e_g = rel_err(dz.cpu().numpy(), OL.block_loss_grad(z_ref, labels))
    log(f"  loss gpu={float(loss.item()):.6f} oracle={L_ref:.6f} rel={e_L:.2e}; row CE rel={e_ce:.2e}; dlogits rel={e_g:.2e}")
    assert P.status() == 0
    assert e_L < tol(cfg) and e_ce < tol(cfg) and e_g < tol(cfg)
