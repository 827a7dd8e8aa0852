"""Pins for the oracle's tiny causal target (no GPU): the verifying forward that the GPU's
dflash_target_forward is compared against.  Pinned to torch's own causal attention, to
causality itself (a prefix's outputs do not depend on what follows), and to the layer taps."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from synth import gen
from oracle import dflash as O
from oracle.tiny_target import TinyTarget


def _target(cfg, n_layers=4):
    m = O.DraftModel(cfg, gen.weights(cfg))
    return TinyTarget(cfg, m, n_layers=n_layers)


def _torch_target(cfg, t, tokens):
    """The target assembled from torch CPU library calls on float64 tensors: F.rms_norm,
    F.linear, F.scaled_dot_product_attention(is_causal=True) with GQA, F.silu; RoPE as a
    multiplication by complex rotations of the pairs (i, i + D/2)."""
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    n = len(tokens)
    D, nq, nkv, H = cfg.head_dim, cfg.n_q, cfg.n_kv, cfg.hidden
    x = T(t.embed)[torch.tensor(tokens)].clone()
    pos = torch.arange(n, dtype=torch.float64)
    freq = torch.exp(-math.log(cfg.rope_theta) * torch.arange(D // 2, dtype=torch.float64) / (D // 2))
    rot = torch.polar(torch.ones(n, D // 2, dtype=torch.float64), pos[:, None] * freq[None])

    def rope_c(u):
        z = torch.complex(u[..., : D // 2], u[..., D // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    hid = []
    for lw in t.layers:
        w = {k: T(v) for k, v in lw.items()}
        a = F.rms_norm(x, (H,), w["in_norm"], eps=cfg.eps)
        q = rope_c(F.rms_norm(F.linear(a, w["wq"]).view(n, nq, D), (D,), w["q_norm"], eps=cfg.eps))
        k = rope_c(F.rms_norm(F.linear(a, w["wk"]).view(n, nkv, D), (D,), w["k_norm"], eps=cfg.eps))
        v = F.linear(a, w["wv"]).view(n, nkv, D)
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                           v.permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)
        x = x + F.linear(o[0].permute(1, 0, 2).reshape(n, nq * D), w["wo"])
        a2 = F.rms_norm(x, (H,), w["post_norm"], eps=cfg.eps)
        x = x + F.linear(F.silu(F.linear(a2, w["w_gate"])) * F.linear(a2, w["w_up"]), w["w_down"])
        hid.append(x.numpy().copy())
    z = F.linear(F.rms_norm(x, (H,), T(t.final_norm), eps=cfg.eps), T(t.lm_head))
    return z.numpy(), hid


@pytest.mark.parametrize("shape", [dict(), dict(n_q=4, n_kv=1), dict(n_q=6, n_kv=3, head_dim=4)])
def test_target_matches_torch_causal_composite(shape):
    cfg = synth.tiny_config(**shape)
    t = _target(cfg)
    tokens = [int(v) for v in gen.tokens(cfg, "pin.target", (11,))]
    z, hid = t.forward(tokens)
    zr, hr = _torch_target(cfg, t, tokens)
    np.testing.assert_allclose(z, zr, rtol=1e-10, atol=1e-10)
    for a, b in zip(hid, hr):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_target_is_causal():
    """Every prefix gives the same outputs at its positions as the whole sequence, and a later
    token changes nothing before it (a missing or reversed mask fails this)."""
    cfg = synth.tiny_config()
    t = _target(cfg)
    tokens = [int(v) for v in gen.tokens(cfg, "pin.causal", (9,))]
    z, hid = t.forward(tokens)
    for n in (1, 4, 8):
        zp, hp = t.forward(tokens[:n])
        np.testing.assert_allclose(zp, z[:n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(hp[-1], hid[-1][:n], rtol=0, atol=1e-12)
    other = tokens[:5] + [(tokens[5] + 1) % cfg.vocab] + tokens[6:]
    z2, _ = t.forward(other)
    np.testing.assert_allclose(z2[:5], z[:5], rtol=0, atol=1e-12)
    assert np.abs(z2[5:] - z[5:]).max() > 1e-6


def test_target_taps_span_shallow_to_deep():
    cfg = synth.tiny_config(n_feat=3)
    t = _target(cfg, n_layers=7)
    assert t.taps == [1, 4, 7]
    tokens = [1, 2, 3]
    _, hid = t.forward(tokens)
    f = t.features(hid)
    assert f.shape == (3, 3, cfg.hidden)
    for i, layer in enumerate(t.taps):
        np.testing.assert_array_equal(f[:, i], hid[layer - 1])
