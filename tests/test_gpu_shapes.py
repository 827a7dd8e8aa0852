"""GPU parity on launch shapes the small cases do not reach: several 64-row GEMM
groups with ragged context lengths (serving concurrency), attention launches with
enough workgroups for the small LDS rings, GQA group 8 at a
32k-token context with a block size that changes per cycle (long chain-of-thought
drafting), tiled GEMMs over 256-row blocks with a half-filled last block, and the
Qwen3-8B-shaped drafter at full size in the launch configuration the benchmark times.
Same bars as the other parity tests."""
import json

import numpy as np
import pytest

import synth
from synth import gen
import oracle

from gpu_support import Pair, log, rel_err, decode, tol, check_draft, assert_draft, run_cycle_case, check_kv_rows, oracle_head

pytestmark = pytest.mark.gpu

# batch 5 x gamma 16 = 80 block rows: one full and one ragged 64-row group; contexts 0..300
MB = synth.Config("mb_bf16", "bf16", hidden=512, n_q=4, n_kv=2, head_dim=128, inter=1024,
                  n_layers=2, n_feat=2, vocab=1000, gamma=16, ctx=300, batch=5, index=79)
# 32 q / 4 kv heads (128 query rows per kv head at gamma 16), 32768-token context
LC = synth.Config("longctx_g8_bf16", "bf16", hidden=512, n_q=32, n_kv=4, head_dim=128, inter=1024,
                  n_layers=2, n_feat=2, vocab=1000, gamma=16, ctx=32768, batch=2, gammas=(16, 8), index=80)
# 8 sequences x 4 kv heads (group 2) at contexts up to 4095: 576 attention workgroups, so
# the 4-stage LDS rings (two workgroups per CU) with 2 query tiles (gamma 16) and 1
# (gamma 8, 4) per workgroup
MR = synth.Config("ring4_bf16", "bf16", hidden=512, n_q=8, n_kv=4, head_dim=128, inter=1024,
                  n_layers=2, n_feat=2, vocab=1000, gamma=16, ctx=4095, batch=8, index=82)
# 8 sequences x 16 kv heads (group 4) at contexts up to 8000: 1024-key attention chunks
# (lengths on both sides of a chunk boundary) in 4-stage rings, with 4 query tiles per
# workgroup at gamma 16, 3 at gamma 11 (the fourth tile is empty), 2 at gamma 6
# (a partly filled tile) and 1 at gamma 3
MT = synth.Config("long_chunks_bf16", "bf16", hidden=512, n_q=64, n_kv=16, head_dim=128, inter=1024,
                  n_layers=1, n_feat=2, vocab=1000, gamma=16, ctx=8000, batch=8, index=83)
# a 250 000-token vocabulary: 7813 LM-head tiles of 32 rows per row at gamma 16 and 4, more than
# the 6144 tile maxima the argmax finish reads in one round, with a partly filled last tile
LV = synth.Config("large_vocab_bf16", "bf16", hidden=512, n_q=4, n_kv=2, head_dim=128, inter=1024,
                  n_layers=1, n_feat=2, vocab=250000, gamma=16, ctx=200, batch=2, index=87)


# 24 sequences x gamma 16 = 384 block rows with a wide SwiGLU (I 11264): the tiled gate|up
# launch has 176 x 3 blocks of 128 rows, so it takes 256-row blocks (eight waves), two of
# them with the second only half filled (rows 384..511 re-read row 383, results dropped);
# at gamma 4 the 96 rows take the weight-streaming kernel
BM = synth.Config("bm256_bf16", "bf16", hidden=512, n_q=4, n_kv=2, head_dim=128, inter=11264,
                  n_layers=1, n_feat=2, vocab=1000, gamma=16, ctx=200, batch=24, index=88)


def test_batch_of_five_ragged_row_groups():
    run_cycle_case(MB, 5, [0, 1, 300, 63, 257], [16, 2, 9], gen.kv_capacity(MB, 64), "mb")


def test_tiled_256_row_blocks_ragged_last_block():
    lengths = [int(x) for x in np.linspace(0, 200, 24)]
    P, _ = run_cycle_case(BM, 24, lengths, [16, 4], gen.kv_capacity(BM, 64), "bm")
    # every sum in the eight-wave blocks runs in a fixed order: two drafts, the same bits
    anchors = gen.tokens(BM, "bm.det", (24,))
    log("case determinism of the 256-row tiled blocks")
    a = P.draft(anchors, 16)
    b = P.draft(anchors, 16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_large_vocabulary_two_finish_rounds():
    run_cycle_case(LV, 2, [0, 200], [16, 4], gen.kv_capacity(LV, 64), "lv")


def test_many_attention_workgroups_small_rings():
    run_cycle_case(MR, 8, [0, 1, 31, 257, 1000, 2047, 3000, 4095], [16, 8, 4], gen.kv_capacity(MR, 64), "mr")


def _draft_inject_cycles(P, gammas, tag):
    cfg, B = P.cfg, P.batch
    for ci, gamma in enumerate(gammas):
        anchors = gen.tokens(cfg, f"{tag}.anchor.{ci}", (B,))
        log(f"  draft cycle {ci} gamma={gamma} len={list(P.okv.len)}")
        got = P.draft(anchors, gamma)
        ref = P.oracle_draft(anchors, gamma)
        m = check_draft(cfg, got, ref, head=oracle_head(P.om))
        log(f"  {json.dumps(m)}")
        assert_draft(cfg, m)
        n_new = (gen.planted_accept(cfg, (B,), gamma, tag=f"{tag}.k.{ci}") + 1).astype(np.int32)
        nf = gen.features(cfg, B, gamma, tag=f"{tag}.feat.{ci}")
        log(f"  inject n_new={list(n_new)}")
        P.inject(nf, n_new)
        P.torch.cuda.synchronize()
        assert P.status() == 0
        assert list(P.cache.len.cpu().numpy()[:B]) == list(P.okv.len)


def test_long_context_group8_dynamic_block():
    cfg = LC
    cap = gen.kv_capacity(cfg, 64)
    log(f"case {cfg.name} lengths=[32768, 20001] cap={cap}")
    P = Pair(cfg, 2, cap, 16)
    P.set_context([32768, 20001], tag="lc")
    _draft_inject_cycles(P, [16, 8, 16], "lc")
    # the rows injected after the long context sit at positions 32768.. and 20001..
    k = decode(P.cache.read_k())
    v = decode(P.cache.read_v())
    lens = P.okv.len
    for b, c0 in enumerate([32768, 20001]):
        check_kv_rows(cfg, k[:, b, :, c0:lens[b]], P.okv.k[:, b, :, c0:lens[b]], v[:, b, :, c0:lens[b]],
                      P.okv.v[:, b, :, c0:lens[b]], f"seq {b} injected rows {c0}..{lens[b]}: ")


def test_long_chunks_ragged_tiles():
    cfg = MT
    cap = gen.kv_capacity(cfg, 64)
    lengths = [8000, 1, 0, 1023, 1024, 1025, 5000, 7777]
    log(f"case {cfg.name} lengths={lengths} cap={cap}")
    P = Pair(cfg, 8, cap, 16)
    P.set_context(lengths, tag="mt")
    _draft_inject_cycles(P, [16, 11, 6, 3], "mt")


def test_qwen3_8b_shape_full_size():
    """Headline shape at full size (H 4096, I 12288, V 151936, 5 layers, context 4096,
    batch 1, gamma 16), with the capacity and launch plans of the benchmark."""
    import torch
    import block_diffusion_drafter_states_amd as dfl
    cfg = synth.get_config("C3")
    cap = (cfg.ctx + 2 * cfg.gamma_max + 63) // 64 * 64        # as in the benchmark
    log(f"case {cfg.name} full size, cap={cap}")
    P = Pair(cfg, 1, cap, cfg.gamma)
    P.set_context([cfg.ctx], tag="full")
    # one cycle's injection: tau = 6 rows at positions 4096..4101 of every layer and kv head
    n_new = np.array([6], dtype=np.int32)
    feat = gen.features(cfg, 1, cfg.gamma, tag="full.feat")
    P.inject(feat, n_new)
    torch.cuda.synchronize()
    assert P.status() == 0 and int(P.cache.len.item()) == cfg.ctx + 6
    k = decode(P.cache.read_k())[:, 0, :, cfg.ctx:cfg.ctx + 6]
    v = decode(P.cache.read_v())[:, 0, :, cfg.ctx:cfg.ctx + 6]
    check_kv_rows(cfg, k, P.okv.k[:, 0, :, cfg.ctx:cfg.ctx + 6], v, P.okv.v[:, 0, :, cfg.ctx:cfg.ctx + 6],
                  "injected rows: ")
    # the draft pass over [4102 context rows ; 16 block rows]
    anchors = gen.tokens(cfg, "full.anchor", (1,))
    got = P.draft(anchors, cfg.gamma)
    ref = P.oracle_draft(anchors, cfg.gamma)
    m = check_draft(cfg, got, ref, head=oracle_head(P.om))
    log(f"  {json.dumps(m)}")
    assert_draft(cfg, m)
    # verify against a planted target, exactly as the benchmark plants it
    d = got[0]
    kpl = np.array([4])
    y = gen.planted_targets(cfg, d, kpl, tag="full.y")
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    com = torch.zeros((1, cfg.gamma), dtype=torch.int32, device="cuda")
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    dfl.verify(torch.as_tensor(d, device="cuda"), torch.as_tensor(y, device="cuda"), acc, com, nxt)
    torch.cuda.synchronize()
    tau, c, n = oracle.verify(d[0], y[0])
    assert acc.item() == tau == 5 and com[0].tolist() == list(c) and nxt.item() == n


def _full_size_cycles(cfg, lengths, gammas, tag, cap=None):
    """Context given directly (seeded K/V rows), then per gamma: draft on both sides,
    compare, and inject a planted number of accepted rows."""
    B = len(lengths)
    cap = cap or (int(max(lengths)) + 2 * cfg.gamma_max + 63) // 64 * 64
    log(f"case {cfg.name} batch={B} lengths {min(lengths)}..{max(lengths)} gammas={gammas} cap={cap}")
    P = Pair(cfg, B, cap, cfg.gamma_max)
    P.set_context(list(lengths), tag=tag)
    _draft_inject_cycles(P, gammas, tag)
    return P


def test_qwen3_4b_shape_tied_head_full_size():
    # H 2560, 32q/8kv, I 9728, V 151936 with the LM head tied to the embedding, context 1024
    cfg = synth.get_config("C2")
    assert cfg.tied
    _full_size_cycles(cfg, [cfg.ctx], [16, 16], "c2full")


def test_llama31_8b_shape_batch32_ragged():
    # full LLaMA-3.1-8B drafter dimensions (I 14336, V 128256) at batch 32: 512 block rows,
    # eight 64-row GEMM groups; contexts ragged in [64, 512] (shorter than the serving
    # workload's), every sequence against the oracle, two cycles
    cfg = synth.get_config("C4").with_(ctx_range=(64, 512))
    lengths = gen.context_lengths(cfg)
    _full_size_cycles(cfg, lengths, [16, 16], "c4full")


def _subset_cycle(cfg, lengths, gamma, sel, tag):
    """The whole batch on the GPU at its full contexts; the oracle for the sequences in
    `sel` only (sequences are independent: each one's drafts, hidden states, logits and
    injected rows depend on its own cache alone).  One draft, then an injection of a planted
    number of rows per sequence, then a second draft over the grown caches."""
    import torch
    B = len(lengths)
    cap = (int(max(lengths)) + 2 * cfg.gamma_max + 63) // 64 * 64
    log(f"case {cfg.name} batch={B} lengths {min(lengths)}..{max(lengths)} gamma={gamma} cap={cap}, "
        f"oracle on sequences {list(sel)} (contexts {[int(lengths[b]) for b in sel]})")
    P = Pair(cfg, B, cap, cfg.gamma_max)
    P.okv = None
    K, V = gen.context_kv(cfg, np.asarray(lengths), cap, tag=tag)
    P.cache.set_context(K, V, lengths)
    okv = oracle.KVCache.from_storage(cfg, K[:, sel], V[:, sel], np.asarray(lengths)[sel])
    del K, V
    sel = list(sel)
    for ci in range(2):
        anchors = gen.tokens(cfg, f"{tag}.anchor.{ci}", (B,))
        d, x, z = P.draft(anchors, gamma)
        ref = [oracle.draft(P.om, okv, i, int(anchors[b]), gamma, return_all=True) for i, b in enumerate(sel)]
        m = check_draft(cfg, (d[sel], x[sel], z[sel]), tuple(np.stack(r) for r in zip(*ref)),
                        head=oracle_head(P.om))
        log(f"  cycle {ci}: {json.dumps(m)}")
        assert_draft(cfg, m)
        if ci == 1:
            break
        n_new = (gen.planted_accept(cfg, (B,), gamma, tag=f"{tag}.k.{ci}") + 1).astype(np.int32)
        nf = gen.features(cfg, B, gamma, tag=f"{tag}.feat.{ci}")
        len0 = P.cache.len.cpu().numpy()[:B].copy()
        P.dfl.inject_kv(P.model, P.cache, P.dev_storage(nf), P.dev_i32(n_new), P.ws)
        torch.cuda.synchronize()
        assert P.status() == 0
        assert list(P.cache.len.cpu().numpy()[:B]) == list(len0 + n_new)
        f = decode(nf)
        for i, b in enumerate(sel):
            oracle.inject(P.om, okv, i, f[b, : int(n_new[b])])
        kk, vv = decode(P.cache.read_k()), decode(P.cache.read_v())
        for i, b in enumerate(sel):
            c0, c1 = int(len0[b]), int(len0[b] + n_new[b])
            check_kv_rows(cfg, kk[:, b, :, c0:c1], okv.k[:, i, :, c0:c1], vv[:, b, :, c0:c1], okv.v[:, i, :, c0:c1],
                          f"seq {b} injected rows {c0}..{c1}: ")
        del kk, vv
    return P


def test_llama31_8b_shape_batch32_serving_contexts():
    """The serving configuration as stated: batch 32, contexts U{512..8192} (1024-key
    attention chunks, 4-stage rings, several refills per chunk), full LLaMA-3.1-8B drafter
    dimensions; the oracle checks the shortest and the longest context and two more."""
    cfg = synth.get_config("C4")
    lengths = gen.context_lengths(cfg)
    order = np.argsort(lengths)
    sel = sorted({int(order[0]), int(order[-1]), 7, 20})
    _subset_cycle(cfg, lengths, 16, sel, "c4serve")


def test_qwen3_8b_shape_batch4_full_size():
    """The Qwen3-8B-shaped drafter at batch 4, context 4096, gamma 16: every sequence."""
    cfg = synth.get_config("C3").with_(batch=4)
    _subset_cycle(cfg, [cfg.ctx] * 4, 16, [0, 1, 2, 3], "c3b4")


def test_coder30b_drafter_shape_32k_context_dynamic_block():
    # H 2048, 32q/4kv (128 query rows per kv head), I 6144, V 151936, batch 8 at a
    # 32768-token context, block size alternating 16 / 8
    cfg = synth.get_config("C5")
    _full_size_cycles(cfg, [cfg.ctx] * cfg.batch, [16, 8], "c5full")


def test_qwen3_8b_shape_prefill_injection():
    """A whole prompt's feature rows at once: the 4096 context positions of the Qwen3-8B
    shape through W_fuse (4096 x 20480) and every layer's W_k | W_v, the many-row GEMM path
    (128 x 128 blocks, 1024 of them for the fusion, 128-byte LDS stages); every written K
    and V row against the oracle, per row."""
    import torch
    cfg = synth.get_config("C3")
    rows = cfg.ctx
    cap = (rows + 2 * cfg.gamma_max + 63) // 64 * 64
    log(f"case {cfg.name} prefill injection of {rows} rows, cap={cap}")
    P = Pair(cfg, 1, cap, rows)
    feat = gen.features(cfg, 1, rows, tag="prefill.feat")
    P.inject(feat, np.array([rows], dtype=np.int32))
    torch.cuda.synchronize()
    assert P.status() == 0 and int(P.cache.len.item()) == rows
    k = decode(P.cache.read_k())[:, 0, :, :rows]
    v = decode(P.cache.read_v())[:, 0, :, :rows]
    check_kv_rows(cfg, k, P.okv.k[:, 0, :, :rows], v, P.okv.v[:, 0, :, :rows], "prefill rows: ")
