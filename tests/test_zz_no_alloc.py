"""dflash_draft_block_noalloc (the library's fixed per-GPU scratch instead of a caller
workspace) against dflash_draft_block on the same inputs, through the C ABI: the same
kernels run on the same data, so drafts, hidden states and logits must agree bit for bit.
Two calls in a row on one GPU, the second with a smaller batch and block: the array keeps
the first call's contents, and nothing of them may leak into the second.  (A call whose
workspace exceeds the array is rejected on the host: test_abi.py.)"""
import numpy as np
import pytest

import synth
from synth import gen

from gpu_support import Pair, log

pytestmark = pytest.mark.gpu

BF = synth.Config("noalloc_bf16", "bf16", hidden=512, n_q=8, n_kv=2, head_dim=128, inter=1024,
                  n_layers=2, n_feat=2, vocab=3000, gamma=16, ctx=700, batch=3, index=91)


def _both(P, anchors, gamma):
    import torch
    import block_diffusion_drafter_states_amd as dfl
    out = []
    for noalloc in (False, True):
        B = len(anchors)
        d = torch.full((B, gamma - 1), -7, dtype=torch.int32, device="cuda")
        hid = torch.full((B, gamma, P.cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        lg = torch.full((B, gamma - 1, P.cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
        a = P.dev_i32(anchors)
        if noalloc:
            dfl.draft_block_noalloc(P.model, P.cache, gamma, a, d, hid, lg)
        else:
            dfl.draft_block(P.model, P.cache, gamma, a, d, P.ws, hid, lg)
        torch.cuda.synchronize()
        out.append((d.cpu().numpy(), hid.cpu().numpy(), lg.cpu().numpy()))
    return out


@pytest.mark.parametrize("cfg", [synth.get_config("C1"), BF], ids=["tiny_f32", "bf16"])
def test_noalloc_matches_workspace_call_twice(cfg):
    lengths = [cfg.ctx, 37, 0][: cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    B = len(lengths)
    cap = gen.kv_capacity(cfg, 64)
    log(f"case {cfg.name} noalloc batch={B} lengths={lengths} cap={cap}")
    P = Pair(cfg, B, cap, cfg.gamma)
    P.set_context(lengths, tag="noalloc")
    # first call: every sequence, full block; second: one sequence, a smaller block
    for call, (nb, gamma) in enumerate([(B, cfg.gamma), (1, max(2, cfg.gamma // 2 - 1))]):
        anchors = gen.tokens(cfg, f"noalloc.anchor.{call}", (nb,))
        (d0, h0, z0), (d1, h1, z1) = _both(P, anchors, gamma)
        log(f"  call {call}: batch {nb} gamma {gamma} drafts {d1.tolist()}")
        assert np.isfinite(h0).all() and np.isfinite(z0).all()
        assert np.array_equal(d0, d1)
        assert np.array_equal(h0.view(np.uint32), h1.view(np.uint32))
        assert np.array_equal(z0.view(np.uint32), z1.view(np.uint32))
    assert P.status() == 0
