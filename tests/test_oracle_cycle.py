"""Pins for the oracle's inject / draft / whole-cycle behaviour (no GPU)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from synth import gen
import oracle
from oracle import dflash as O
from oracle.tiny_target import TinyTarget, greedy
from oracle.spec import spec_decode, OracleDrafter, ConstantDrafter, CorruptedGreedyDrafter


def _model(cfg, overrides=None):
    return O.DraftModel(cfg, gen.weights(cfg, overrides))


# ----------------------------------------------------------------------------- losslessness

@pytest.mark.parametrize("gamma", [2, 4, 8])
@pytest.mark.parametrize("kind", ["oracle", "constant", "corrupted"])
def test_spec_decode_is_lossless(gamma, kind):
    cfg = synth.tiny_config(gamma=gamma)
    m = _model(cfg)
    t = TinyTarget(cfg, m)
    prompt = [3, 1, 4, 1, 5, 9]
    ref = greedy(t, prompt, 24)
    drafter = {"oracle": lambda: OracleDrafter(m, 128),
               "constant": lambda: ConstantDrafter(ref[1]),
               "corrupted": lambda: CorruptedGreedyDrafter(t, seed=gamma, p_corrupt=0.3)}[kind]()
    out, taus = spec_decode(t, drafter, prompt, 24, gamma)
    assert out == ref
    assert all(1 <= x <= gamma for x in taus)
    if kind == "corrupted" and gamma > 2:
        assert max(taus) > 1          # the mock produces real partial acceptances


def test_spec_decode_bf16_drafter_is_lossless():
    cfg = synth.tiny_config(dtype="bf16", gamma=4)
    m = _model(cfg)
    t = TinyTarget(cfg, m)
    prompt = [2, 7, 1, 8]
    ref = greedy(t, prompt, 16)
    out, _ = spec_decode(t, OracleDrafter(m, 64), prompt, 16, 4)
    assert out == ref


# ----------------------------------------------------------------------------- injection

def _kv_from_injection(cfg, m, feats, chunks, cap=64):
    kv = O.KVCache(cfg, 1, cap)
    lo = 0
    for n in chunks:
        O.inject(m, kv, 0, feats[lo:lo + n])
        lo += n
    return kv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_injection_chunking_invariance(dtype):
    cfg = synth.tiny_config(dtype=dtype)
    m = _model(cfg)
    feats = O.decode_storage(gen.features(cfg, 1, 12)[0])
    a = _kv_from_injection(cfg, m, feats, [12])
    b = _kv_from_injection(cfg, m, feats, [3, 1, 8])
    c = _kv_from_injection(cfg, m, feats, [1] * 12)
    for other in (b, c):
        assert list(other.len) == [12]
        np.testing.assert_allclose(other.k, a.k, rtol=0, atol=1e-12)
        np.testing.assert_allclose(other.v, a.v, rtol=0, atol=1e-12)


def test_injection_len_and_untouched_rows():
    cfg = synth.tiny_config()
    m = _model(cfg)
    kv = O.KVCache(cfg, 2, 32)
    feats = O.decode_storage(gen.features(cfg, 2, 5))
    O.inject(m, kv, 1, feats[1, :5])
    O.inject(m, kv, 0, feats[0, :0])
    assert list(kv.len) == [0, 5]
    assert not kv.k[:, 0].any() and not kv.k[:, 1, :, 5:].any()
    assert kv.k[:, 1, :, :5].any()
    with pytest.raises(ValueError):
        O.inject(m, kv, 1, O.decode_storage(gen.features(cfg, 1, 28))[0])


def test_injected_keys_are_rotated_at_their_positions():
    # A row injected at position p equals the same row injected at position 0, rotated by p.
    cfg = synth.tiny_config()
    m = _model(cfg)
    f = O.decode_storage(gen.features(cfg, 1, 1))[0]
    kv0 = O.KVCache(cfg, 1, 16)
    O.inject(m, kv0, 0, f)
    kv5 = O.KVCache(cfg, 1, 16)
    kv5.len[0] = 5
    O.inject(m, kv5, 0, f)
    k0 = kv0.k[:, 0, :, 0, :]           # [L][n_kv][D] at position 0 (rotation = identity)
    k5 = kv5.k[:, 0, :, 5, :]
    # rope() rotates axis -3 by the given positions: here one position (5) per layer row
    np.testing.assert_allclose(O.rope(k0, np.full(cfg.n_layers, 5.0), cfg.rope_theta), k5,
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(kv0.v[:, 0, :, 0], kv5.v[:, 0, :, 5])


# ----------------------------------------------------------------------------- draft structure

def test_draft_without_sublayer_outputs_is_embedding_lookup():
    # W_o = 0 and W_down = 0: the residual stream never changes, so every mask row
    # drafts argmax(W_lm rms(E[MASK])) and the hidden output is the embedding rows.
    cfg = synth.tiny_config()
    ov = {}
    for l in range(cfg.n_layers):
        ov[f"layers.{l}.wo"] = np.zeros((cfg.hidden, cfg.n_q * cfg.head_dim), np.float32)
        ov[f"layers.{l}.w_down"] = np.zeros((cfg.hidden, cfg.inter), np.float32)
    m = _model(cfg, ov)
    kv = O.KVCache(cfg, 1, 32)
    O.inject(m, kv, 0, O.decode_storage(gen.features(cfg, 1, 4))[0])
    d, x, z = O.draft(m, kv, 0, 5, cfg.gamma, return_all=True)
    np.testing.assert_array_equal(x[0], m.embed[5])
    np.testing.assert_array_equal(x[1:], np.broadcast_to(m.embed[cfg.mask_id], x[1:].shape))
    e = m.embed[cfg.mask_id]
    zz = m.lm_head @ (e / np.sqrt(np.mean(e * e) + cfg.eps) * m.final_norm)
    assert (d == int(np.argmax(zz))).all()


def test_draft_block_is_bidirectional():
    # The anchor row (first in the block) must see the mask rows that follow it:
    # changing the mask embedding changes the anchor row's output.
    cfg = synth.tiny_config()
    m1 = _model(cfg)
    m2 = _model(cfg)
    m2.embed = m2.embed.copy()
    m2.embed[cfg.mask_id] *= -1.0
    m2.lm_head = m2.embed if cfg.tied else m2.lm_head
    kv = O.KVCache(cfg, 1, 32)
    O.inject(m1, kv, 0, O.decode_storage(gen.features(cfg, 1, 3))[0])
    _, x1, _ = O.draft(m1, kv, 0, 2, cfg.gamma, return_all=True)
    _, x2, _ = O.draft(m2, kv, 0, 2, cfg.gamma, return_all=True)
    assert np.abs(x1[0] - x2[0]).max() > 1e-6


def test_draft_depends_on_every_layers_injected_context():
    # KV injection into every layer: perturbing only the last layer's cached context
    # values changes the output.
    cfg = synth.tiny_config()
    m = _model(cfg)
    kv = O.KVCache(cfg, 1, 32)
    O.inject(m, kv, 0, O.decode_storage(gen.features(cfg, 1, 6))[0])
    _, x1, _ = O.draft(m, kv, 0, 1, cfg.gamma, return_all=True)
    kv.v[-1, 0, :, :6] += 1.0
    _, x2, _ = O.draft(m, kv, 0, 1, cfg.gamma, return_all=True)
    assert np.abs(x1 - x2).max() > 1e-6


def _torch_draft(cfg, m, kv, anchor, gamma):
    """The same drafter assembled from torch CPU library calls (F.rms_norm, F.linear,
    F.scaled_dot_product_attention with GQA, F.silu) on float64 tensors, in f32
    configurations (no bf16 rounding).  RoPE is the complex-number form."""
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    C = int(kv.len[0])
    D, nq, nkv, H = cfg.head_dim, cfg.n_q, cfg.n_kv, cfg.hidden
    ids = torch.tensor([anchor] + [cfg.mask_id] * (gamma - 1))
    x = T(m.embed)[ids].clone()
    pos = torch.arange(C, C + gamma, dtype=torch.float64)
    freq = torch.exp(-math.log(cfg.rope_theta) * torch.arange(D // 2, dtype=torch.float64) / (D // 2))
    rot = torch.polar(torch.ones(gamma, D // 2, dtype=torch.float64), pos[:, None] * freq[None])

    def rope_c(t):  # t [G][h][D]
        z = torch.complex(t[..., : D // 2], t[..., D // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    for l, lw in enumerate(m.layers):
        w = {k: T(v) for k, v in lw.items()}
        a = F.rms_norm(x, (H,), w["in_norm"], eps=cfg.eps)
        q = F.rms_norm(F.linear(a, w["wq"]).view(gamma, nq, D), (D,), w["q_norm"], eps=cfg.eps)
        k = F.rms_norm(F.linear(a, w["wk"]).view(gamma, nkv, D), (D,), w["k_norm"], eps=cfg.eps)
        v = F.linear(a, w["wv"]).view(gamma, nkv, D)
        q, k = rope_c(q), rope_c(k)
        kk = torch.cat([T(kv.k[l, 0, :, :C]), k.permute(1, 0, 2)], 1)[None]
        vv = torch.cat([T(kv.v[l, 0, :, :C]), v.permute(1, 0, 2)], 1)[None]
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], kk, vv, enable_gqa=True)
        x = x + F.linear(o[0].permute(1, 0, 2).reshape(gamma, nq * D), w["wo"])
        a2 = F.rms_norm(x, (H,), w["post_norm"], eps=cfg.eps)
        x = x + F.linear(F.silu(F.linear(a2, w["w_gate"])) * F.linear(a2, w["w_up"]), w["w_down"])
    z = F.linear(F.rms_norm(x[1:], (H,), T(m.final_norm), eps=cfg.eps), T(m.lm_head))
    return x.numpy(), z.numpy()


@pytest.mark.parametrize("shape", [dict(), dict(n_q=4, n_kv=1), dict(n_q=6, n_kv=3, head_dim=4)])
def test_draft_matches_torch_library_composite(shape):
    cfg = synth.tiny_config(**shape)
    m = _model(cfg)
    kv = O.KVCache(cfg, 1, 32)
    O.inject(m, kv, 0, O.decode_storage(gen.features(cfg, 1, 7))[0])
    d, x, z = O.draft(m, kv, 0, 9, cfg.gamma, return_all=True)
    xr, zr = _torch_draft(cfg, m, kv, 9, cfg.gamma)
    np.testing.assert_allclose(x, xr, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(z, zr, rtol=1e-10, atol=1e-10)


def test_draft_bf16_rounds_only_at_contract_points():
    # With every weight bf16-exact, the bf16 oracle differs from the unrounded
    # computation by a small relative amount (the A-operand / q,k,v roundings),
    # not by O(1): a rounding at a wrong place (e.g. the residual) would still pass
    # this, but a missing norm scale or wrong operand would not.
    cfg_b = synth.tiny_config(dtype="bf16")
    cfg_f = cfg_b.with_(dtype="f32")
    W = gen.weights(cfg_b)
    mb = O.DraftModel(cfg_b, W)
    mf = O.DraftModel(cfg_f, W)
    kvb = O.KVCache(cfg_b, 1, 32)
    kvf = O.KVCache(cfg_f, 1, 32)
    f = O.decode_storage(gen.features(cfg_b, 1, 5))[0]
    O.inject(mb, kvb, 0, f)
    O.inject(mf, kvf, 0, f)
    _, xb, zb = O.draft(mb, kvb, 0, 3, cfg_b.gamma, return_all=True)
    _, xf, zf = O.draft(mf, kvf, 0, 3, cfg_b.gamma, return_all=True)
    rel = np.linalg.norm(zb - zf) / np.linalg.norm(zf)
    assert 1e-5 < rel < 3e-2
    # cache rows are bf16-exact
    assert np.array_equal(O.round_bf16(kvb.k), kvb.k)


def test_cycle_runs_inject_draft_verify_per_sequence():
    cfg = synth.tiny_config(batch=2)
    m = _model(cfg)
    kv = O.KVCache(cfg, 2, 32)
    kv.len[:] = [0, 3]
    feat = O.decode_storage(gen.features(cfg, 2, cfg.gamma))
    # target agrees with the drafts for 2 positions on sequence 0, none on sequence 1
    def target(b, d):
        y = np.array([(t + 1) % cfg.vocab for t in d] + [0])
        if b == 0:
            y[:2] = d[:2]
        return y
    out = O.cycle(m, kv, feat, [4, 1], [5, 6], cfg.gamma, target)
    assert list(out["accept_len"]) == [3, 1]
    assert list(kv.len) == [4, 4]
