"""Pins for where the oracle rounds to bf16, and for the injected K/V of every layer (no GPU).

The precision contract puts the bf16 rounding rho at fixed points of the cycle: every GEMM
input (the fused features, each layer's normalised rows, the attention output, the SwiGLU
product, the final normalised rows), the q / k / v vectors after their norm and rotation,
and the K / V rows written into the cache; the residual stream, norms, softmax and all sums
stay unrounded.  The tests below rebuild injection and drafting from torch CPU library
routines (F.linear, F.rms_norm, F.scaled_dot_product_attention with GQA, F.silu, RoPE as a
complex rotation) in float64 and put rho exactly at those points, in the order the pages'
steps reach them.  The oracle's own rho calls are recorded: at every contract point the
composite's value before rounding must equal the one the oracle rounded there (to float64
noise) and the composite continues from the oracle's rounded value, so that the two sides
are compared point by point without independent rounding decisions (two computations that
differ by float noise may round a value lying on a bf16 tie differently).  A rounding
added, dropped or moved (for example of the residual stream, or of a GEMM output), or an
operand rounded before instead of after its norm, changes the sequence of rounded values
and fails.  The rounding function itself is pinned to torch's float32 -> bfloat16
conversion in test_oracle_primitives.py."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from synth import gen
from oracle import dflash as O

T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


class RhoTape:
    """Records the oracle's rounding calls (input, output) in order."""

    def __init__(self, m):
        self.calls = []
        inner = m.num.rho

        def rec(x):
            y = inner(x)
            self.calls.append((np.array(x, dtype=np.float64, copy=True), np.array(y, dtype=np.float64, copy=True)))
            return y
        m.num.rho = rec


class Replay:
    """The composite's rho: check the value against the oracle's next rounding call and
    continue from the oracle's rounded value."""

    def __init__(self, calls, bf16):
        self.calls = list(calls)
        self.i = 0
        self.bf16 = bf16

    def __call__(self, t, what):
        assert self.i < len(self.calls), f"composite rounds {what} after the oracle's last rounding"
        xin, yout = self.calls[self.i]
        self.i += 1
        got = t.detach().numpy().reshape(xin.shape) if t.numel() == xin.size else None
        assert got is not None, f"{what}: shape {tuple(t.shape)} vs the oracle's {xin.shape}"
        np.testing.assert_allclose(got, xin, rtol=1e-11, atol=1e-12, err_msg=f"value before rounding {what}")
        if self.bf16:
            # bf16-exact, within half an ulp of the input (8 significant bits)
            assert np.array_equal(O.round_bf16(yout), yout)
            assert (np.abs(yout - xin) <= np.abs(xin) * 2.0 ** -8 + 1e-300).all()
        else:
            assert np.array_equal(yout, xin)
        return T(yout).reshape(t.shape)

    def done(self):
        assert self.i == len(self.calls), f"the oracle rounded {len(self.calls) - self.i} more values"


def _rope_c(t, pos, theta):
    """Rotate-half RoPE as a complex rotation; t [P][h][D], positions pos [P]."""
    D = t.shape[-1]
    freq = torch.exp(-math.log(theta) * torch.arange(D // 2, dtype=torch.float64) / (D // 2))
    rot = torch.polar(torch.ones(len(pos), D // 2, dtype=torch.float64),
                      torch.as_tensor(pos, dtype=torch.float64)[:, None] * freq[None])
    z = torch.complex(t[..., : D // 2], t[..., D // 2:]) * rot[:, None, :]
    return torch.cat([z.real, z.imag], -1)


def _torch_inject(cfg, m, feat_rows, C, rho, shared_norm=None):
    """K, V rows [L][n][n_kv][D] of feature rows [n][F][H] injected at positions C.., all layers."""
    n, H, D, nkv = feat_rows.shape[0], cfg.hidden, cfg.head_dim, cfg.n_kv
    u = rho(T(feat_rows).reshape(n, -1), "fused features")
    c = F.linear(u, T(m.w_fuse))
    if shared_norm is not None:
        c = F.rms_norm(c, (H,), T(shared_norm), eps=cfg.eps)
    pos = np.arange(C, C + n)
    ks, vs = [], []
    for lw in m.layers:
        w = {k: T(v) for k, v in lw.items()}
        ch = rho(F.rms_norm(c, (H,), w["in_norm"], eps=cfg.eps), "context rows (input norm)")
        k = F.rms_norm(F.linear(ch, w["wk"]).view(n, nkv, D), (D,), w["k_norm"], eps=cfg.eps)
        v = F.linear(ch, w["wv"]).view(n, nkv, D)
        ks.append(rho(_rope_c(k, pos, cfg.rope_theta), "context k"))
        vs.append(rho(v, "context v"))
    return torch.stack(ks), torch.stack(vs)


def _torch_draft(cfg, m, kv, b, anchor, gamma, rho):
    C = int(kv.len[b])
    D, nq, nkv, H = cfg.head_dim, cfg.n_q, cfg.n_kv, cfg.hidden
    ids = torch.tensor([anchor] + [cfg.mask_id] * (gamma - 1))
    x = T(m.embed)[ids].clone()
    pos = np.arange(C, C + gamma)
    for l, lw in enumerate(m.layers):
        w = {k: T(v) for k, v in lw.items()}
        a = rho(F.rms_norm(x, (H,), w["in_norm"], eps=cfg.eps), f"layer {l} input rows")
        q = F.rms_norm(F.linear(a, w["wq"]).view(gamma, nq, D), (D,), w["q_norm"], eps=cfg.eps)
        k = F.rms_norm(F.linear(a, w["wk"]).view(gamma, nkv, D), (D,), w["k_norm"], eps=cfg.eps)
        v = F.linear(a, w["wv"]).view(gamma, nkv, D)
        q = rho(_rope_c(q, pos, cfg.rope_theta), f"layer {l} q")
        k = rho(_rope_c(k, pos, cfg.rope_theta), f"layer {l} k")
        v = rho(v, f"layer {l} v")
        kk = torch.cat([T(kv.k[l, b, :, :C]), k.permute(1, 0, 2)], 1)[None]
        vv = torch.cat([T(kv.v[l, b, :, :C]), v.permute(1, 0, 2)], 1)[None]
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], kk, vv, enable_gqa=True)
        o = rho(o[0].permute(1, 0, 2).reshape(gamma, nq * D), f"layer {l} attention output")
        x = x + F.linear(o, w["wo"])
        a2 = rho(F.rms_norm(x, (H,), w["post_norm"], eps=cfg.eps), f"layer {l} MLP input rows")
        h = rho(F.silu(F.linear(a2, w["w_gate"])) * F.linear(a2, w["w_up"]), f"layer {l} SwiGLU product")
        x = x + F.linear(h, w["w_down"])
    zr = rho(F.rms_norm(x[1:], (H,), T(m.final_norm), eps=cfg.eps), "final rows")
    return x, F.linear(zr, T(m.lm_head))


SHAPES = [dict(), dict(n_q=4, n_kv=1), dict(n_q=6, n_kv=3, head_dim=4, n_layers=3)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_injection_of_every_layer_matches_torch_composite(dtype, shape):
    cfg = synth.tiny_config(dtype=dtype, **shape)
    m = O.DraftModel(cfg, gen.weights(cfg))
    tape = RhoTape(m)
    kv = O.KVCache(cfg, 1, 32)
    kv.len[0] = 3
    feats = O.decode_storage(gen.features(cfg, 1, 6, tag="roundpin"))[0]
    O.inject(m, kv, 0, feats)
    rep = Replay(tape.calls, dtype == "bf16")
    k, v = _torch_inject(cfg, m, feats, 3, rep)
    rep.done()
    # every layer's injected rows (the cache stores [n_kv][position][D])
    np.testing.assert_array_equal(kv.k[:, 0, :, 3:9], k.permute(0, 2, 1, 3).numpy())
    np.testing.assert_array_equal(kv.v[:, 0, :, 3:9], v.permute(0, 2, 1, 3).numpy())
    assert not kv.k[:, 0, :, :3].any() and not kv.k[:, 0, :, 9:].any()
    if dtype == "bf16":
        assert len(tape.calls) == 1 + 3 * cfg.n_layers


def test_injection_with_shared_fusion_norm_matches_composite():
    """The alternative reading (one shared RMSNorm right after W_fuse) is exercised too: it
    equals the composite with that norm, and differs from the default reading."""
    cfg = synth.tiny_config(dtype="bf16")
    W = gen.weights(cfg)
    m = O.DraftModel(cfg, W)
    shared = 1.0 + 0.1 * np.random.default_rng(5).standard_normal(cfg.hidden)
    tape = RhoTape(m)
    kv = O.KVCache(cfg, 1, 16)
    feats = O.decode_storage(gen.features(cfg, 1, 4, tag="shared"))[0]
    O.inject(m, kv, 0, feats, shared_fuse_norm=shared)
    rep = Replay(tape.calls, True)
    k, v = _torch_inject(cfg, m, feats, 0, rep, shared_norm=shared)
    rep.done()
    np.testing.assert_array_equal(kv.k[:, 0, :, :4], k.permute(0, 2, 1, 3).numpy())
    np.testing.assert_array_equal(kv.v[:, 0, :, :4], v.permute(0, 2, 1, 3).numpy())
    kv2 = O.KVCache(cfg, 1, 16)
    O.inject(O.DraftModel(cfg, W), kv2, 0, feats)
    assert np.abs(kv2.k - kv.k).max() > 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("ctx", [0, 5])
def test_draft_rounds_exactly_at_the_contract_points(dtype, shape, ctx):
    cfg = synth.tiny_config(dtype=dtype, **shape)
    m = O.DraftModel(cfg, gen.weights(cfg))
    kv = O.KVCache(cfg, 1, 32)
    if ctx:
        O.inject(m, kv, 0, O.decode_storage(gen.features(cfg, 1, ctx, tag="roundctx"))[0])
    tape = RhoTape(m)
    d, x, z = O.draft(m, kv, 0, 7, cfg.gamma, return_all=True)
    rep = Replay(tape.calls, dtype == "bf16")
    xr, zr = _torch_draft(cfg, m, kv, 0, 7, cfg.gamma, rep)
    rep.done()
    assert len(tape.calls) == 7 * cfg.n_layers + 1
    np.testing.assert_allclose(x, xr.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(z, zr.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_array_equal(d, O.argmax_lowest(zr.numpy()))


def test_composite_detects_a_misplaced_rounding():
    """The replay check is not vacuous: a composite that rounds one more value (the residual
    stream after the attention block) disagrees with the oracle's sequence of roundings."""
    cfg = synth.tiny_config(dtype="bf16")
    m = O.DraftModel(cfg, gen.weights(cfg))
    kv = O.KVCache(cfg, 1, 32)
    O.inject(m, kv, 0, O.decode_storage(gen.features(cfg, 1, 3, tag="mis"))[0])
    tape = RhoTape(m)
    O.draft(m, kv, 0, 7, cfg.gamma)
    rep = Replay(tape.calls, True)
    orig_linear = F.linear
    state = {"n": 0}

    def linear_rounding_wo(a, w):   # the 4th linear of layer 0 is W_o: round its output too
        y = orig_linear(a, w)
        state["n"] += 1
        if state["n"] == 4:
            y = rep(y, "misplaced: W_o output")
        return y
    F.linear = linear_rounding_wo
    try:
        with pytest.raises(AssertionError):
            _torch_draft(cfg, m, kv, 0, 7, cfg.gamma, rep)
    finally:
        F.linear = orig_linear
