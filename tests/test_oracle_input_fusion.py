"""Pins for the oracle's input-fusion conditioning (the alternative that KV injection is
measured against, "DFlash" technical summary sections 2.2 and 4)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from synth import gen
from oracle import dflash as O
from oracle.input_fusion import inject_input_fusion


def _setup(cfg, batch=2, cap=128, ctx=(5, 0)):
    m = O.DraftModel(cfg, gen.weights(cfg))
    kv = O.KVCache(cfg, batch, cap)
    for b, n in enumerate(ctx):
        if n:
            O.inject(m, kv, b, O.decode_storage(gen.features(cfg, 1, n, tag=f"if.ctx{b}"))[0])
    return m, kv


def _copy(kv):
    c = O.KVCache.__new__(O.KVCache)
    c.k, c.v, c.len, c.cap = kv.k.copy(), kv.v.copy(), kv.len.copy(), kv.cap
    return c


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_first_layer_kv_equals_kv_injection(dtype):
    """Layer 0's K/V of a context row are W_k / W_v of the fused feature in both conditionings."""
    cfg = synth.tiny_config(gamma=8).with_(dtype=dtype)
    m, kv = _setup(cfg)
    feat = O.decode_storage(gen.features(cfg, 1, 6, tag="if.new"))[0]
    a, b_ = _copy(kv), _copy(kv)
    inject_input_fusion(m, a, 0, feat)
    O.inject(m, b_, 0, feat)
    C = int(kv.len[0])
    np.testing.assert_allclose(a.k[0, 0, :, C:C + 6], b_.k[0, 0, :, C:C + 6], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a.v[0, 0, :, C:C + 6], b_.v[0, 0, :, C:C + 6], rtol=0, atol=1e-12)
    assert a.len[0] == b_.len[0] == C + 6
    # deeper layers see hidden states that went through the layers below: they differ
    assert np.abs(a.k[1, 0, :, C:C + 6] - b_.k[1, 0, :, C:C + 6]).max() > 1e-3


def test_chunked_equals_whole():
    """Context rows are causal: appending them in pieces gives the same cache."""
    cfg = synth.tiny_config(gamma=8)
    m, kv = _setup(cfg)
    feat = O.decode_storage(gen.features(cfg, 1, 7, tag="if.chunk"))[0]
    a, b_ = _copy(kv), _copy(kv)
    inject_input_fusion(m, a, 1, feat)
    inject_input_fusion(m, b_, 1, feat[:3])
    inject_input_fusion(m, b_, 1, feat[3:4])
    inject_input_fusion(m, b_, 1, feat[4:])
    np.testing.assert_allclose(a.k, b_.k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a.v, b_.v, rtol=0, atol=1e-12)
    assert list(a.len) == list(b_.len)


def test_equals_torch_causal_composite():
    """From an empty cache (fp32 configuration: no rounding), the rows' final hidden states
    and every layer's K/V equal a composite of torch CPU library calls: F.rms_norm,
    F.linear, F.scaled_dot_product_attention(is_causal=True, enable_gqa=True), F.silu;
    RoPE as a multiplication by complex rotations of the pairs (i, i + D/2)."""
    cfg = synth.tiny_config(gamma=8)
    m, kv = _setup(cfg, batch=1, ctx=(0,))
    n = 9
    feat = O.decode_storage(gen.features(cfg, 1, n, tag="if.torch"))[0]
    x_ref = inject_input_fusion(m, kv, 0, feat)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    D, nq, nkv, H = cfg.head_dim, cfg.n_q, cfg.n_kv, cfg.hidden
    x = F.linear(T(feat.reshape(n, -1)), T(m.w_fuse))
    pos = torch.arange(n, dtype=torch.float64)
    freq = torch.exp(-math.log(cfg.rope_theta) * torch.arange(D // 2, dtype=torch.float64) / (D // 2))
    rot = torch.polar(torch.ones(n, D // 2, dtype=torch.float64), pos[:, None] * freq[None])

    def rope_c(u):
        z = torch.complex(u[..., : D // 2], u[..., D // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    for l, lw in enumerate(m.layers):
        w = {k: T(v) for k, v in lw.items()}
        a = F.rms_norm(x, (H,), w["in_norm"], eps=cfg.eps)
        q = rope_c(F.rms_norm(F.linear(a, w["wq"]).view(n, nq, D), (D,), w["q_norm"], eps=cfg.eps))
        k = rope_c(F.rms_norm(F.linear(a, w["wk"]).view(n, nkv, D), (D,), w["k_norm"], eps=cfg.eps))
        v = F.linear(a, w["wv"]).view(n, nkv, D)
        np.testing.assert_allclose(kv.k[l, 0, :, :n], k.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(kv.v[l, 0, :, :n], v.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-10)
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                           v.permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)
        x = x + F.linear(o[0].permute(1, 0, 2).reshape(n, nq * D), w["wo"])
        a2 = F.rms_norm(x, (H,), w["post_norm"], eps=cfg.eps)
        x = x + F.linear(F.silu(F.linear(a2, w["w_gate"])) * F.linear(a2, w["w_up"]), w["w_down"])
    np.testing.assert_allclose(x_ref, x.numpy(), rtol=1e-9, atol=1e-9)


def test_later_rows_do_not_change_earlier_ones():
    cfg = synth.tiny_config(gamma=8)
    m, kv = _setup(cfg)
    feat = O.decode_storage(gen.features(cfg, 1, 6, tag="if.causal"))[0]
    feat2 = feat.copy()
    feat2[4:] += 1.0
    a, b_ = _copy(kv), _copy(kv)
    xa = inject_input_fusion(m, a, 0, feat)
    xb = inject_input_fusion(m, b_, 0, feat2)
    C = int(kv.len[0])
    np.testing.assert_array_equal(xa[:4], xb[:4])
    np.testing.assert_array_equal(a.k[:, 0, :, C:C + 4], b_.k[:, 0, :, C:C + 4])
    assert np.abs(xa[4:] - xb[4:]).max() > 1e-3
