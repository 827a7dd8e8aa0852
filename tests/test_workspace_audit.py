"""Host-only check of the launch plans against the workspace layout (no GPU needed).

For the five workload shapes at batch 1, 4, 8 and 32 (capped at what the shape holds in
memory on one GPU), block sizes 16, 8 and 2, and injections of one block's rows and of a
whole prompt, `dflash_audit_workspace` runs the launch sequences of injection, input
fusion, drafting, the block loss and the verifying target's forward without launching
anything, and checks that every workspace range a kernel writes (computed from the
launch's own arguments and grid) stays inside the region the layout carved for it.  A
workspace overrun in the carving (the kind a plan with more tiles than its region would
cause) shows up here as a violation."""
import ctypes

import pytest

from block_diffusion_drafter_states_amd import _abi
from block_diffusion_drafter_states_amd._abi import dflash_config, DFLASH_OK
import synth

from test_abi import _lib


def _config(c, batch, cap, gmax):
    return dflash_config(hidden=c.hidden, n_q_heads=c.n_q, n_kv_heads=c.n_kv, head_dim=c.head_dim,
                         inter=c.inter, n_layers=c.n_layers, n_feat=c.n_feat, vocab=c.vocab, gamma_max=gmax,
                         mask_token_id=c.mask_id, max_batch=batch, kv_capacity=cap, rms_eps=c.eps,
                         dtype=_abi.DFLASH_BF16 if c.dtype == "bf16" else _abi.DFLASH_F32)


def _audit(L, cfg, batch, gamma, rows):
    n = [ctypes.c_int32(-1) for _ in range(3)]
    rc = L.dflash_audit_workspace(ctypes.byref(cfg), batch, gamma, rows, *[ctypes.byref(x) for x in n])
    return rc, [x.value for x in n]


CASES = [(name, b) for name in ("C1", "C2", "C3", "C4", "C5") for b in (1, 4, 8, 32)]


@pytest.mark.parametrize("name,batch", CASES)
def test_every_launch_writes_inside_its_region(name, batch):
    L = _lib()
    c = synth.get_config(name)
    gmax = c.gamma_max
    cap = (c.max_ctx + 2 * gmax + 63) // 64 * 64
    cfg = _config(c, batch, cap, gmax)
    for gamma in sorted({gmax, 8, 2} & set(range(2, gmax + 1))):
        for rows in sorted({gmax, 1, 7} | ({c.ctx} if batch == 1 else set())):
            rc, (launches, writes, bad) = _audit(L, cfg, batch, gamma, rows)
            assert rc == DFLASH_OK, (name, batch, gamma, rows, rc)
            assert launches > 0 and writes > launches // 2
            assert bad == 0, f"{name} batch {batch} gamma {gamma} rows {rows}: {bad} of {writes} writes outside"


def test_audit_counts_grow_with_layers():
    """Every layer's launches are audited: doubling the drafter's depth adds launches and
    audited writes, and the layout stays consistent."""
    L = _lib()
    c = synth.get_config("C1")
    cfg = _config(c, 1, 128, c.gamma)
    rc1, n1 = _audit(L, cfg, 1, c.gamma, 8)
    rc2, n2 = _audit(L, _config(c.with_(n_layers=4), 1, 128, c.gamma), 1, c.gamma, 8)
    assert rc1 == rc2 == DFLASH_OK
    assert n1[2] == n2[2] == 0
    assert n2[0] > n1[0] and n2[1] > n1[1]


def test_audit_validates_arguments():
    L = _lib()
    c = synth.get_config("C1")
    cfg = _config(c, 2, 128, c.gamma)
    assert _audit(L, cfg, 3, c.gamma, 8)[0] == _abi.DFLASH_EINVAL          # batch > max_batch
    assert _audit(L, cfg, 1, c.gamma + 1, 8)[0] == _abi.DFLASH_EINVAL      # gamma > gamma_max
    assert _audit(L, cfg, 1, 1, 8)[0] == _abi.DFLASH_EINVAL
    assert _audit(L, cfg, 1, c.gamma, 0)[0] == _abi.DFLASH_EINVAL
    bad = _config(c.with_(head_dim=32), 1, 128, c.gamma)
    assert _audit(L, bad, 1, c.gamma, 8)[0] == _abi.DFLASH_EUNSUPPORTED
    n = ctypes.c_int32()
    assert L.dflash_audit_workspace(ctypes.byref(cfg), 1, c.gamma, 8, None, ctypes.byref(n),
                                    ctypes.byref(n)) == _abi.DFLASH_EINVAL
