"""Pins for the oracle's building blocks against library routines, closed forms
and invariants (no GPU).  Each check is chosen so that a plausible slip in the
oracle (a dropped scale, a wrong sign, a swapped operand, a wrong head mapping)
fails it."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import dflash as O

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_on_fp32_inputs():
    x = RNG.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # plant exact ties (the 16 dropped bits are 0x8000) with both parities of the kept lsb
    u = x.view(np.uint32).copy()
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[1000:1500] = (u[1000:1500] & np.uint32(0xFFFE0000)) | np.uint32(0x18000)
    x = u.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_closed_forms():
    # 1 + 2**-8 is the midpoint between 1 and 1 + 2**-7: ties to even -> 1
    assert O.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2**-8 is the midpoint between 1+2**-7 and 1+2**-6: ties to even -> 1 + 2**-6
    assert O.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert O.round_bf16(np.array([-(1 + 2 ** -7 + 2 ** -20)]))[0] == -(1 + 2 ** -7)
    assert O.round_bf16(np.array([0.0]))[0] == 0.0
    # carry into the exponent: just below 2 rounds up to 2
    assert O.round_bf16(np.array([2 - 2 ** -10]))[0] == 2.0


def test_decode_storage_bf16_bits():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000], dtype=np.uint16)
    assert list(O.decode_storage(bits)) == [1.0, -1.0, 3.140625, 0.0]


# ----------------------------------------------------------------------------- norms, activations, linear

def test_rms_norm_matches_torch():
    x = RNG.standard_normal((7, 96))
    w = 1 + 0.1 * RNG.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_silu_matches_torch():
    x = RNG.standard_normal(1000) * 5
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-15)


def test_linear_matches_torch():
    a = RNG.standard_normal((5, 33))
    w = RNG.standard_normal((17, 33))
    np.testing.assert_allclose(O.linear(a, w), F.linear(torch.from_numpy(a), torch.from_numpy(w)).numpy(),
                               rtol=1e-12, atol=1e-12)


def test_argmax_ties_lowest_index():
    z = np.array([[0.5, 2.0, 2.0, 1.0], [3.0, 3.0, 3.0, 3.0], [-1.0, -2.0, -1.0, -3.0]])
    assert list(O.argmax_lowest(z)) == [1, 0, 0]


# ----------------------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((1, 3, 16))
    np.testing.assert_array_equal(O.rope(x, np.array([0]), 1e6), x)


def test_rope_two_dims_closed_form():
    # D = 2: one pair, angle = p; (1, 0) rotates to (cos p, sin p); (0, 1) to (-sin p, cos p)
    x = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])            # [P=2][H=1][2]
    p = np.array([0.7, 2.5])
    got = O.rope(x, p, 10000.0)
    np.testing.assert_allclose(got[0, 0], [math.cos(0.7), math.sin(0.7)], rtol=1e-15)
    np.testing.assert_allclose(got[1, 0], [-math.sin(2.5), math.cos(2.5)], rtol=1e-15)


def test_rope_equals_complex_rotation():
    # rotate-half pairs (x_i, x_{i+D/2}) form z_i = x_i + i x_{i+D/2}; RoPE multiplies z_i by e^{i a_i}
    D, theta = 32, 1e6
    x = RNG.standard_normal((5, 2, D))
    p = np.array([0, 1, 17, 4096, 32767])
    got = O.rope(x, p, theta)
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    freq = np.exp(-np.log(theta) * (np.arange(D // 2) / (D // 2)))
    rot = z * np.exp(1j * p[:, None, None] * freq[None, None, :])
    np.testing.assert_allclose(got[..., : D // 2], rot.real, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(got[..., D // 2:], rot.imag, rtol=1e-9, atol=1e-12)


def test_rope_preserves_pair_norms_and_is_relative():
    D = 64
    q = RNG.standard_normal((1, 1, D))
    k = RNG.standard_normal((1, 1, D))
    r = O.rope(q, np.array([123]), 1e6)
    n0 = q[..., : D // 2] ** 2 + q[..., D // 2:] ** 2
    n1 = r[..., : D // 2] ** 2 + r[..., D // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # dot products depend only on the position difference
    s1 = (O.rope(q, np.array([10]), 1e6) * O.rope(k, np.array([3]), 1e6)).sum()
    s2 = (O.rope(q, np.array([1010]), 1e6) * O.rope(k, np.array([1003]), 1e6)).sum()
    np.testing.assert_allclose(s1, s2, rtol=1e-10)


# ----------------------------------------------------------------------------- attention

def _sdpa(q, k, v, gqa=True):
    """torch SDPA reference: q [G][n_q][D], k/v [T][n_kv][D] -> [G][n_q][D]."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=False, enable_gqa=gqa)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n_q,n_kv", [(4, 2), (8, 8), (8, 1), (6, 3)])
def test_attention_zero_context_is_block_self_attention(n_q, n_kv):
    G, D = 5, 16
    q = RNG.standard_normal((G, n_q, D))
    k = RNG.standard_normal((G, n_kv, D))
    v = RNG.standard_normal((G, n_kv, D))
    empty = np.zeros((n_kv, 0, D))
    got = O.block_attention(q, empty, empty, k, v)
    np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C", [1, 7, 40])
def test_attention_with_context_matches_sdpa_over_concat(C):
    G, n_q, n_kv, D = 4, 6, 2, 8
    q = RNG.standard_normal((G, n_q, D))
    kc = RNG.standard_normal((n_kv, C, D))
    vc = RNG.standard_normal((n_kv, C, D))
    kb = RNG.standard_normal((G, n_kv, D))
    vb = RNG.standard_normal((G, n_kv, D))
    got = O.block_attention(q, kc, vc, kb, vb)
    kk = np.concatenate([kc.transpose(1, 0, 2), kb], 0)
    vv = np.concatenate([vc.transpose(1, 0, 2), vb], 0)
    np.testing.assert_allclose(got, _sdpa(q, kk, vv), rtol=1e-11, atol=1e-12)


def test_attention_brute_force_loops():
    G, n_q, n_kv, D, C = 3, 4, 2, 4, 3
    q = RNG.standard_normal((G, n_q, D))
    kc = RNG.standard_normal((n_kv, C, D)); vc = RNG.standard_normal((n_kv, C, D))
    kb = RNG.standard_normal((G, n_kv, D)); vb = RNG.standard_normal((G, n_kv, D))
    got = O.block_attention(q, kc, vc, kb, vb)
    g = n_q // n_kv
    for j in range(G):
        for h in range(n_q):
            hk = h // g
            keys = [kc[hk, t] for t in range(C)] + [kb[t, hk] for t in range(G)]
            vals = [vc[hk, t] for t in range(C)] + [vb[t, hk] for t in range(G)]
            s = [sum(q[j, h, d] * kk[d] for d in range(D)) / math.sqrt(D) for kk in keys]
            mx = max(s)
            e = [math.exp(si - mx) for si in s]
            tot = sum(e)
            for d in range(D):
                ref = sum(e[t] * vals[t][d] for t in range(len(keys))) / tot
                assert abs(got[j, h, d] - ref) < 1e-12


def test_attention_mha_and_mqa_equal_explicit_head_repetition():
    G, D, C = 4, 8, 6
    for n_q, n_kv in [(4, 4), (4, 1)]:
        q = RNG.standard_normal((G, n_q, D))
        kc = RNG.standard_normal((n_kv, C, D)); vc = RNG.standard_normal((n_kv, C, D))
        kb = RNG.standard_normal((G, n_kv, D)); vb = RNG.standard_normal((G, n_kv, D))
        got = O.block_attention(q, kc, vc, kb, vb)
        rep = n_q // n_kv
        got_rep = O.block_attention(q, np.repeat(kc, rep, 0), np.repeat(vc, rep, 0),
                                    np.repeat(kb, rep, 1), np.repeat(vb, rep, 1))
        np.testing.assert_allclose(got, got_rep, rtol=1e-13, atol=1e-14)


def test_attention_context_permutation_invariance():
    G, n_q, n_kv, D, C = 3, 4, 2, 8, 11
    q = RNG.standard_normal((G, n_q, D))
    kc = RNG.standard_normal((n_kv, C, D)); vc = RNG.standard_normal((n_kv, C, D))
    kb = RNG.standard_normal((G, n_kv, D)); vb = RNG.standard_normal((G, n_kv, D))
    perm = RNG.permutation(C)
    a = O.block_attention(q, kc, vc, kb, vb)
    b = O.block_attention(q, kc[:, perm], vc[:, perm], kb, vb)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_attention_zero_query_is_mean_of_values():
    # q = 0 gives equal scores: the output is the plain mean of all C + G value rows
    G, n_q, n_kv, D, C = 3, 4, 2, 8, 5
    q = np.zeros((G, n_q, D))
    kc = RNG.standard_normal((n_kv, C, D)); vc = RNG.standard_normal((n_kv, C, D))
    kb = RNG.standard_normal((G, n_kv, D)); vb = RNG.standard_normal((G, n_kv, D))
    got = O.block_attention(q, kc, vc, kb, vb)
    for h in range(n_q):
        hk = h // (n_q // n_kv)
        mean = (vc[hk].sum(0) + vb[:, hk].sum(0)) / (C + G)
        np.testing.assert_allclose(got[:, h], np.broadcast_to(mean, (G, D)), rtol=1e-12)


def test_attention_split_context_lse_merge_equals_whole():
    # Attention over a context split in chunks, merged by log-sum-exp weights, equals
    # attention over the whole context: the identity the GPU's split-K relies on.
    G, n_q, n_kv, D, C = 4, 4, 2, 8, 37
    q = RNG.standard_normal((G, n_q, D))
    kc = RNG.standard_normal((n_kv, C, D)); vc = RNG.standard_normal((n_kv, C, D))
    kb = RNG.standard_normal((G, n_kv, D)); vb = RNG.standard_normal((G, n_kv, D))
    whole = O.block_attention(q, kc, vc, kb, vb)
    keys = [np.concatenate([kc[h], kb[:, h]], 0) for h in range(n_kv)]
    vals = [np.concatenate([vc[h], vb[:, h]], 0) for h in range(n_kv)]
    bounds = [0, 5, 6, 20, C + G]
    g = n_q // n_kv
    for h in range(n_q):
        ms, ls, os_ = [], [], []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            s = q[:, h] @ keys[h // g][lo:hi].T / math.sqrt(D)
            m = s.max(1, keepdims=True)
            e = np.exp(s - m)
            ms.append(m); ls.append(e.sum(1, keepdims=True)); os_.append(e @ vals[h // g][lo:hi])
        M = np.max(np.concatenate(ms, 1), 1, keepdims=True)
        num = sum(np.exp(m - M) * o for m, o in zip(ms, os_))
        den = sum(np.exp(m - M) * l for m, l in zip(ms, ls))
        np.testing.assert_allclose(num / den, whole[:, h], rtol=1e-12, atol=1e-13)
