"""GPU parity of the verifying target's forward (dflash_target_forward / dflash_advance_len)
against the oracle's tiny causal target: a prompt processed in chunks, then two verification
blocks with only an accepted prefix kept in between.  Same error bars as the drafter's tests
(relative L2 error of logits and features; argmax checked as in check_draft)."""
import json

import numpy as np
import pytest

import synth
from synth import gen
from oracle import dflash as O
from oracle.tiny_target import TinyTarget

from gpu_support import log, decode, tol, check_draft

pytestmark = pytest.mark.gpu

TB = synth.Config("target_bf16", "bf16", hidden=512, n_q=8, n_kv=2, head_dim=128, inter=1024,
                  n_layers=2, n_feat=3, vocab=1000, gamma=8, ctx=64, batch=2, index=81)


def _case(cfg, batch, prompt_len, gammas, taus, n_target_layers=4):
    import torch
    import block_diffusion_drafter_states_amd as dfl
    W_d = gen.weights(cfg)
    om = O.DraftModel(cfg, W_d)
    tt = TinyTarget(cfg, om, n_layers=n_target_layers)
    tcfg = cfg.with_(n_layers=n_target_layers)
    W_t = gen.weights(tcfg.with_(index=cfg.index + 1000))          # the tiny target's own weights
    cap = (prompt_len + sum(gammas) + 2 * cfg.gamma_max + 63) // 64 * 64
    drafter = dfl.Model(cfg, W_d, device="cuda", max_batch=batch, kv_capacity=cap)
    target = dfl.Model(tcfg, W_t, device="cuda", max_batch=batch, kv_capacity=cap, share_from=drafter)
    cache = dfl.Cache(target)
    ws = dfl.Workspace(target, batch, 0)
    taps = tt.taps
    F = len(taps)
    seqs = [list(gen.tokens(cfg, f"tgt.prompt.{b}", (prompt_len,))) for b in range(batch)]
    log(f"case {cfg.name} target layers {n_target_layers} taps {taps} batch {batch} prompt {prompt_len} "
        f"gammas {gammas} taus {taus} cap {cap}")

    def run(rows_tokens):
        """One target_forward over rows_tokens [B][rows] (list of lists); returns y, feat, logits."""
        rows = len(rows_tokens[0])
        tok = torch.as_tensor(np.asarray(rows_tokens, dtype=np.int32), device="cuda")
        y = torch.full((batch, rows), -1, dtype=torch.int32, device="cuda")
        feat = torch.zeros((batch, rows, F, cfg.hidden), dtype=target.storage_dtype, device="cuda")
        lg = torch.full((batch, rows, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
        dfl.target_forward(target, cache, tok, y, ws, feat=feat, taps=taps, dbg_logits=lg)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        return y.cpu().numpy(), decode(dfl.to_storage(feat)), lg.cpu().numpy()

    def oracle(b, start, rows):
        logits, hiddens = tt.forward(seqs[b])
        feat = tt.storage_features(hiddens)               # what the drafter's injection reads
        return logits[start:start + rows], np.asarray(feat[start:start + rows], dtype=np.float64)

    def compare(tag, y, feat, lg, start, rows):
        ref_lg, ref_feat = zip(*[oracle(b, start, rows) for b in range(batch)])
        ref_lg, ref_feat = np.stack(ref_lg), np.stack(ref_feat)
        ref_y = np.argmax(ref_lg, axis=-1)
        m = check_draft(cfg, (y, feat.reshape(batch, rows, -1), lg), (ref_y, ref_feat.reshape(batch, rows, -1), ref_lg))
        m["feat_rel"] = m.pop("hidden_rel")
        m["feat_row_max"] = m.pop("hidden_row_max")
        log(f"  {tag} rows {start}..{start + rows}: {json.dumps(m)}")
        assert m["feat_rel"] < tol(cfg) and m["logits_rel"] < tol(cfg)
        assert m["feat_row_max"] < tol(cfg) and m["logits_row_max"] < tol(cfg)
        assert m["argmax_self_mismatch"] == 0 and m["wide_mismatch"] == 0 and m["not_near_optimal"] == 0
        if cfg.dtype == "f32":
            assert m["strict_mismatch"] == 0

    # the prompt, in chunks of at most gamma_max rows, each kept whole
    pos = 0
    while pos < prompt_len:
        rows = min(cfg.gamma_max, prompt_len - pos)
        y, feat, lg = run([s[pos:pos + rows] for s in seqs])
        compare("prompt", y, feat, lg, pos, rows)
        dfl.advance_len(target, cache, torch.full((batch,), rows, dtype=torch.int32, device="cuda"))
        pos += rows
    # verification blocks: gamma fresh tokens per sequence, then keep only tau of them
    for ci, (gamma, tau) in enumerate(zip(gammas, taus)):
        block = [list(gen.tokens(cfg, f"tgt.block.{ci}.{b}", (gamma,))) for b in range(batch)]
        for b in range(batch):
            seqs[b] = seqs[b] + block[b]
        y, feat, lg = run(block)
        compare(f"block {ci}", y, feat, lg, pos, gamma)
        dfl.advance_len(target, cache, torch.full((batch,), tau, dtype=torch.int32, device="cuda"))
        for b in range(batch):
            seqs[b] = seqs[b][:pos + tau]
        pos += tau
        assert list(cache.len.cpu().numpy()[:batch]) == [pos] * batch


def test_target_forward_f32_matches_tiny_target():
    _case(synth.get_config("C1"), 1, 20, [8, 8, 5], [3, 8, 1])


def test_target_forward_bf16_batch2_matches_tiny_target():
    _case(TB, 2, 37, [8, 6], [5, 2])
