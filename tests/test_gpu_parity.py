"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.  Bars: verify outputs and draft tokens bit-exact (draft tokens
only where the oracle's top-2 logit gap is >= 1e-2); K/V cache, hidden and
logits within rel-err 1e-4 (fp32 storage) / 2e-2 (bf16 storage)."""
import json
import os

import numpy as np
import pytest

import synth
from synth import gen
import oracle
from oracle import dflash as O

from gpu_support import Pair, log, rel_err, decode, tol, check_draft, assert_draft, run_cycle_case, oracle_head

pytestmark = pytest.mark.gpu

C1 = synth.get_config("C1")
# bf16 shape with several tiles per GEMM, a ragged vocabulary tile (1000 = 7*128 + 104),
# a ragged attention chunk, g = 2 and head_dim 128
MINI = synth.Config("mini_bf16", "bf16", hidden=512, n_q=4, n_kv=2, head_dim=128, inter=1024,
                    n_layers=2, n_feat=2, vocab=1000, gamma=16, ctx=300, batch=2, index=77)
# GQA group 8 (128 query rows per kv head at gamma 16: eight query tiles in one workgroup)
G8 = synth.Config("g8_bf16", "bf16", hidden=512, n_q=8, n_kv=1, head_dim=128, inter=512,
                  n_layers=1, n_feat=2, vocab=512, gamma=16, ctx=700, batch=1, index=78)


def test_c1_fp32_cycles():
    run_cycle_case(C1, 1, [C1.ctx], [8, 8, 4, 2], gen.kv_capacity(C1, 64), "c1")


def test_mini_bf16_ragged_batch_and_empty_context():
    run_cycle_case(MINI, 2, [300, 0], [16, 9, 2], gen.kv_capacity(MINI, 64), "mini")


def test_group8_two_query_groups():
    run_cycle_case(G8, 1, [700], [16, 8], gen.kv_capacity(G8, 64), "g8")


def test_draft_is_deterministic():
    cfg = MINI
    P = Pair(cfg, 2, gen.kv_capacity(cfg, 64), 16)
    P.set_context([257, 40])
    anchors = [3, 999]
    log("case determinism mini_bf16")
    a = P.draft(anchors, 16)
    b = P.draft(anchors, 16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_draft_against_synthetic_context_cache():
    # context K/V given directly (not through injection): isolates the draft pass
    cfg = MINI
    P = Pair(cfg, 2, gen.kv_capacity(cfg, 256), 16)      # 300 + 16 + 256 -> 576 rows
    P.set_context([511, 129], tag="ctx2")
    anchors = [5, 6]
    log("case synthetic context mini_bf16")
    got = P.draft(anchors, 16)
    ref = P.oracle_draft(anchors, 16)
    m = check_draft(cfg, got, ref, head=oracle_head(P.om))
    log(f"  {json.dumps(m)}")
    assert_draft(cfg, m)


def test_verify_matches_oracle_bit_exact():
    import torch
    import block_diffusion_drafter_states_amd as dfl
    cfg = synth.get_config("C3")
    rng = np.random.default_rng(5)
    for gamma, B in [(2, 3), (8, 5), (16, 64), (16, 1), (100, 4)]:
        log(f"case verify gamma={gamma} batch={B}")
        d = rng.integers(0, cfg.vocab, size=(B, gamma - 1)).astype(np.int32)
        k = rng.integers(0, gamma, size=B)
        y = gen.planted_targets(cfg, d, k, tag=f"v{gamma}.{B}")
        dd, yy = torch.as_tensor(d, device="cuda"), torch.as_tensor(y, device="cuda")
        acc = torch.zeros(B, dtype=torch.int32, device="cuda")
        com = torch.zeros((B, gamma), dtype=torch.int32, device="cuda")
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        dfl.verify(dd, yy, acc, com, nxt)
        torch.cuda.synchronize()
        for b in range(B):
            tau, c, n = oracle.verify(d[b], y[b])
            assert acc[b].item() == tau == k[b] + 1
            assert list(com[b].cpu().numpy()) == list(c)
            assert nxt[b].item() == n


def test_verify_golden_cases_on_gpu():
    import torch
    import block_diffusion_drafter_states_amd as dfl
    path = os.path.join(os.path.dirname(__file__), "golden", "verify_cases.json")
    for c in json.load(open(path))["cases"]:
        log(f"case verify golden {c['name']}")
        G = len(c["target"])
        dd = torch.tensor([c["draft"]], dtype=torch.int32, device="cuda")
        yy = torch.tensor([c["target"]], dtype=torch.int32, device="cuda")
        acc = torch.zeros(1, dtype=torch.int32, device="cuda")
        com = torch.zeros((1, G), dtype=torch.int32, device="cuda")
        nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
        dfl.verify(dd, yy, acc, com, nxt)
        torch.cuda.synchronize()
        assert acc.item() == c["accept_len"]
        assert com[0].tolist() == c["committed"]
        assert nxt.item() == c["next_anchor"]


def test_device_status_flags_and_no_partial_writes():
    cfg = C1
    cap = gen.kv_capacity(cfg)          # ctx + gamma rounded to 64
    P = Pair(cfg, 1, cap, 64)
    feat = gen.features(cfg, 1, 64, tag="ovf")
    log("case overflow: inject more rows than the capacity allows")
    P.set_context([cap - 3])
    before_k = P.cache.read_k().copy()
    P.dfl.inject_kv(P.model, P.cache, P.dev_storage(feat[:, :8]), P.dev_i32([8]), P.ws)
    P.torch.cuda.synchronize()
    assert P.status() & P.dfl.STATUS_KV_OVERFLOW
    assert P.cache.len.item() == cap - 3
    assert np.array_equal(P.cache.read_k(), before_k)
    log("case bad count: n_new > rows_stride")
    P.cache.status.zero_()
    P.set_context([5])
    P.dfl.inject_kv(P.model, P.cache, P.dev_storage(feat[:, :4]), P.dev_i32([9]), P.ws)
    P.torch.cuda.synchronize()
    assert P.status() & P.dfl.STATUS_BAD_COUNT
    assert P.cache.len.item() == 5
    log("case bad anchor id")
    P.cache.status.zero_()
    P.draft([cfg.vocab + 5], 8)
    assert P.status() & P.dfl.STATUS_BAD_TOKEN
