"""End-to-end speculative decoding on the GPU, every step through the C ABI: the target's
forward over the prompt (its tapped features injected into the drafter), then cycles of
draft -> the target's forward over [anchor ; drafts] -> greedy verify -> inject the accepted
rows' features -> advance the target's cache.  Greedy verification is lossless ("DFlash"
technical summary, §1 and the speculative-decoding background): the tokens produced must be
the oracle target's plain greedy decode.  Where GPU and oracle part ways, the oracle's own
top-2 gap at that step must be a near-tie that rounding can flip, and only the shared prefix
is compared.

Two draft sources: the GPU drafter itself (random weights: drafts mostly rejected), and
planted drafts (the oracle's greedy continuation with seeded corruptions), which make the
loop take partial acceptances of every length.  With ``policy`` the block size of every
cycle is chosen by dflash_choose_gamma from the accept lengths so far and a cost table."""
import numpy as np
import pytest

import synth
from synth import gen
from oracle import dflash as O
from oracle.tiny_target import TinyTarget, greedy

from gpu_support import log, top2_gap

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-3          # fp32 storage: logit errors are ~1e-6 of the logits' scale


def _spec_loop(cfg, batch, prompt_len, gamma, n_tokens, mode, n_target_layers=4, seed=5, policy=None):
    import torch
    import block_diffusion_drafter_states_amd as dfl
    dev = "cuda"
    W_d = gen.weights(cfg)
    om = O.DraftModel(cfg, W_d)
    tt = TinyTarget(cfg, om, n_layers=n_target_layers)
    tcfg = cfg.with_(n_layers=n_target_layers)
    W_t = gen.weights(tcfg.with_(index=cfg.index + 1000))
    prompts = [list(gen.tokens(cfg, f"spec.prompt.{b}", (prompt_len,))) for b in range(batch)]
    refs = [greedy(tt, p, n_tokens + gamma) for p in prompts]
    cap = (prompt_len + n_tokens + 2 * gamma + 63) // 64 * 64
    drafter = dfl.Model(cfg, W_d, device=dev, max_batch=batch, kv_capacity=cap)
    target = dfl.Model(tcfg, W_t, device=dev, max_batch=batch, kv_capacity=cap, share_from=drafter)
    dcache, tcache = dfl.Cache(drafter), dfl.Cache(target)
    gmax = cfg.gamma_max
    ws_d = dfl.Workspace(drafter, batch, gmax)
    ws_t = dfl.Workspace(target, batch, 0)
    taps, F, H = tt.taps, len(tt.taps), cfg.hidden
    log(f"spec loop {cfg.name} mode {mode} batch {batch} prompt {prompt_len} gamma {gamma} tokens {n_tokens}")

    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32), device=dev).contiguous()

    # prompt: the target's forward in chunks of at most gamma_max rows, each chunk's features injected
    pos = 0
    while pos < prompt_len:
        rows = min(gmax, prompt_len - pos)
        tok = i32([p[pos:pos + rows] for p in prompts])
        y = torch.empty((batch, rows), dtype=torch.int32, device=dev)
        feat = torch.empty((batch, rows, F, H), dtype=target.storage_dtype, device=dev)
        dfl.target_forward(target, tcache, tok, y, ws_t, feat=feat, taps=taps)
        n = i32([rows] * batch)
        dfl.inject_kv(drafter, dcache, feat, n, ws_d)
        dfl.advance_len(target, tcache, n)
        pos += rows
    anchor = y[:, -1].contiguous()
    out = [[int(t)] for t in anchor.cpu().numpy()]

    rng = np.random.default_rng(seed)
    tau = torch.empty((batch,), dtype=torch.int32, device=dev)
    nxt = torch.empty((batch,), dtype=torch.int32, device=dev)
    taus, used = [], []
    hist_t, hist_g = [], []
    while min(len(o) for o in out) < n_tokens:
        if policy is not None:             # block size of this cycle from the accept lengths so far
            gamma, _ = dfl.choose_gamma(hist_t[-64:], hist_g[-64:], policy, 2, gmax)
        used.append(gamma)
        d = torch.empty((batch, gamma - 1), dtype=torch.int32, device=dev)
        y = torch.empty((batch, gamma), dtype=torch.int32, device=dev)
        feat = torch.empty((batch, gamma, F, H), dtype=target.storage_dtype, device=dev)
        committed = torch.empty((batch, gamma), dtype=torch.int32, device=dev)
        if mode == "drafter":
            dfl.draft_block(drafter, dcache, gamma, anchor, d, ws_d)
        else:
            plant = []
            for b in range(batch):
                cont = list(refs[b][len(out[b]):len(out[b]) + gamma - 1])
                for j in range(gamma - 1):
                    if rng.random() < 0.25:
                        cont[j] = (cont[j] + 1) % cfg.vocab
                plant.append(cont)
            d.copy_(i32(plant))
        tok = torch.cat([anchor[:, None], d], dim=1).contiguous()
        dfl.target_forward(target, tcache, tok, y, ws_t, feat=feat, taps=taps)
        dfl.verify(d, y, tau, committed, nxt)
        dfl.inject_kv(drafter, dcache, feat, tau, ws_d)
        dfl.advance_len(target, tcache, tau)
        anchor = nxt.clone()
        torch.cuda.synchronize()
        assert int(tcache.status.item()) == 0 and int(dcache.status.item()) == 0
        t_h, c_h = tau.cpu().numpy(), committed.cpu().numpy()
        for b in range(batch):
            out[b].extend(int(v) for v in c_h[b, :t_h[b]])
        taus.append([int(v) for v in t_h])
        hist_t.extend(int(v) for v in t_h)
        hist_g.extend([gamma] * batch)
    assert list(tcache.len.cpu().numpy()[:batch]) == list(dcache.len.cpu().numpy()[:batch])
    log(f"  cycles {len(taus)} block sizes {used} accept lengths {taus}")

    for b in range(batch):
        got, ref = out[b][:n_tokens], refs[b][:n_tokens]
        if got == ref:
            continue
        i = next(k for k in range(n_tokens) if got[k] != ref[k])
        logits, _ = tt.forward(prompts[b] + ref[:i])
        gap = float(top2_gap(logits[-1]))
        log(f"  seq {b}: first difference at token {i} (oracle top-2 gap {gap:.3e})")
        assert gap < NEAR_TIE, f"sequence {b} differs from greedy decoding at token {i}"
    return (taus, used) if policy is not None else taus


def test_spec_loop_gpu_drafter_is_lossless():
    _spec_loop(synth.get_config("C1"), 2, 13, 8, 40, "drafter")


def test_spec_loop_planted_partial_acceptances_is_lossless():
    taus = _spec_loop(synth.get_config("C1"), 2, 13, 8, 48, "planted")
    flat = [t for row in taus for t in row]
    assert max(flat) > 1 and min(flat) < 8        # partial acceptances actually happened


def test_spec_loop_with_block_size_policy_is_lossless():
    """Block size per cycle from dflash_choose_gamma with a cost table affine in the block size,
    steep enough that the choice follows the acceptance estimate (6 at p = 0.8, 5 at 0.75, 4 at
    0.7): the loop changes its block size and stays lossless."""
    cfg = synth.get_config("C1")
    cost = [0.0, 0.0] + [300.0 + 50.0 * g for g in range(2, cfg.gamma_max + 1)]
    taus, used = _spec_loop(cfg, 2, 13, 8, 56, "planted", seed=9, policy=cost)
    assert len(set(used)) > 1            # the policy moved the block size
    assert all(2 <= g <= cfg.gamma_max for g in used)
