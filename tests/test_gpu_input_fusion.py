"""GPU parity of input-fusion conditioning (dflash_inject_kv_input_fusion: every draft layer
runs over the fused context rows and keeps their K/V) against the oracle, and of the
drafting pass that reads the resulting cache; ragged row counts, a second injection on
top of the first, and the count / capacity checks."""
import json

import numpy as np
import pytest

import synth
from synth import gen
from oracle.input_fusion import inject_input_fusion

from gpu_support import Pair, log, rel_err, decode, tol, check_draft, assert_draft, check_kv_rows, oracle_head

pytestmark = pytest.mark.gpu

MINI = synth.Config("if_mini_bf16", "bf16", hidden=512, n_q=8, n_kv=2, head_dim=128, inter=1024,
                    n_layers=3, n_feat=2, vocab=1000, gamma=16, ctx=120, batch=3, index=86)


def _inject(P, rows, n_new, tag):
    import torch
    cfg, B = P.cfg, P.batch
    feat = gen.features(cfg, B, rows, tag=tag)
    before = list(P.okv.len)
    P.dfl.inject_kv_input_fusion(P.model, P.cache, P.dev_storage(feat), P.dev_i32(n_new), P.ws)
    torch.cuda.synchronize()
    f = decode(feat)
    for b in range(B):
        inject_input_fusion(P.om, P.okv, b, f[b, :int(n_new[b])])
    assert P.status() == 0
    assert list(P.cache.len.cpu().numpy()[:B]) == list(P.okv.len)
    k, v = decode(P.cache.read_k()), decode(P.cache.read_v())
    for b in range(B):
        c0, c1 = before[b], int(P.okv.len[b])
        if c1 == c0:
            continue
        check_kv_rows(cfg, k[:, b, :, c0:c1], P.okv.k[:, b, :, c0:c1], v[:, b, :, c0:c1], P.okv.v[:, b, :, c0:c1],
                      f"{tag} seq {b} rows {c0}..{c1}: ")


def _draft(P, gamma, tag):
    anchors = gen.tokens(P.cfg, f"{tag}.anchor", (P.batch,))
    got = P.draft(anchors, gamma)
    ref = P.oracle_draft(anchors, gamma)
    m = check_draft(P.cfg, got, ref, head=oracle_head(P.om))
    log(f"  draft gamma={gamma}: {json.dumps(m)}")
    assert_draft(P.cfg, m)


def test_input_fusion_fp32_tiny():
    cfg = synth.get_config("C1")
    P = Pair(cfg, 1, gen.kv_capacity(cfg, 64), 16)
    P.set_context([cfg.ctx], tag="if.c1")
    _inject(P, 8, [5], "if.c1.a")
    _inject(P, 8, [8], "if.c1.b")
    _draft(P, cfg.gamma, "if.c1")


def test_input_fusion_bf16_ragged_then_draft():
    cfg = MINI
    P = Pair(cfg, 3, gen.kv_capacity(cfg, 64), 16)
    P.set_context([0, 120, 17], tag="if.mini")
    _inject(P, 16, [16, 1, 6], "if.mini.a")
    _inject(P, 7, [0, 7, 3], "if.mini.b")
    _draft(P, 16, "if.mini")
    _draft(P, 5, "if.mini5")


def test_input_fusion_count_and_capacity_checks():
    import torch
    cfg = MINI
    cap = gen.kv_capacity(cfg, 64)            # 120 + 16 + 64 -> 256
    P = Pair(cfg, 2, cap, 16)
    P.set_context([10, cap - 8], tag="if.chk")
    feat = P.dev_storage(gen.features(cfg, 2, 16, tag="if.chk.f"))
    # n_new above rows_stride: status bit, len unchanged for that sequence only
    P.dfl.inject_kv_input_fusion(P.model, P.cache, feat[:, :4].contiguous(), P.dev_i32([5, 0]), P.ws)
    torch.cuda.synchronize()
    assert P.status() & P.dfl._abi.STATUS_BAD_COUNT
    assert list(P.cache.len.cpu().numpy()[:2]) == [10, cap - 8]
    P.cache.status.zero_()
    # 16 rows from len cap - 8 do not fit: overflow bit, len unchanged; the other sequence advances
    P.dfl.inject_kv_input_fusion(P.model, P.cache, feat, P.dev_i32([3, 2]), P.ws)
    torch.cuda.synchronize()
    assert P.status() & P.dfl._abi.STATUS_KV_OVERFLOW
    assert list(P.cache.len.cpu().numpy()[:2]) == [13, cap - 8]
