"""The C-ABI library loads, exports every symbol include/dflash.h declares, its
ctypes structs match the header, and every host-detectable error returns its
code without touching a device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from block_diffusion_drafter_states_amd import _abi
from block_diffusion_drafter_states_amd._abi import (dflash_config, dflash_kv, dflash_layer_weights, dflash_weights,
                                                     dflash_trace, DFLASH_EINVAL, DFLASH_EUNSUPPORTED,
                                                     DFLASH_EWORKSPACE)
import synth
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def _lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libdflash.so not built (run __graft_entry__.build())")
    return _abi.lib()


def _header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    assert _header_functions() == sorted(_abi.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in _header_functions():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {_abi.LIB_PATH}").read()
    for name in _header_functions():
        assert re.search(rf"\bT {name}\b", out), name


def _struct_fields(name):
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    end = re.search(r"\}\s*" + name + ";", txt).start()
    body = txt[txt.rindex("typedef struct {", 0, end) + len("typedef struct {"):end]
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        names = decl.split()[-1] if "," not in decl else None
        if names is None:
            # "const void *in_norm, *wq, ..." style
            parts = decl.split(",")
            first = parts[0].split()[-1].lstrip("*")
            fields += [first] + [p.strip().lstrip("*") for p in parts[1:]]
        else:
            fields.append(names.lstrip("*"))
    return fields


@pytest.mark.parametrize("cname,pyt", [("dflash_config", dflash_config), ("dflash_layer_weights", dflash_layer_weights),
                                       ("dflash_weights", dflash_weights), ("dflash_kv", dflash_kv),
                                       ("dflash_trace", dflash_trace)])
def test_ctypes_structs_match_header(cname, pyt):
    assert _struct_fields(cname) == [f[0] for f in pyt._fields_]


def _cfg(**kw):
    c = synth.get_config("C1")
    d = dict(hidden=c.hidden, n_q_heads=c.n_q, n_kv_heads=c.n_kv, head_dim=c.head_dim, inter=c.inter,
             n_layers=c.n_layers, n_feat=c.n_feat, vocab=c.vocab, gamma_max=c.gamma, mask_token_id=c.mask_id,
             max_batch=1, kv_capacity=128, rms_eps=1e-6, dtype=0)
    d.update(kw)
    return dflash_config(**d)


def test_workspace_bytes_validates_config():
    L = _lib()
    ok = L.dflash_workspace_bytes(ctypes.byref(_cfg()), 1, 16)
    assert ok > 0
    assert L.dflash_workspace_bytes(ctypes.byref(_cfg()), 2, 16) == 0          # batch > max_batch
    assert L.dflash_workspace_bytes(ctypes.byref(_cfg(head_dim=128)), 1, 16) == 0   # fp32 needs D=64
    assert L.dflash_workspace_bytes(ctypes.byref(_cfg(gamma_max=17)), 1, 16) == 0
    assert L.dflash_workspace_bytes(ctypes.byref(_cfg(kv_capacity=100)), 1, 16) == 0
    assert L.dflash_workspace_bytes(ctypes.byref(_cfg(dtype=7)), 1, 16) == 0
    assert L.dflash_workspace_bytes(None, 1, 16) == 0
    bf = _cfg(dtype=1, head_dim=128, n_q_heads=4, n_kv_heads=2, hidden=512, inter=512)
    assert L.dflash_workspace_bytes(ctypes.byref(bf), 1, 16) > 0


FAKE = 0x1000   # never dereferenced: every call below fails validation first


def _weights(L_layers=2, null_field=None):
    arr = (dflash_layer_weights * L_layers)()
    for l in range(L_layers):
        for f, _ in dflash_layer_weights._fields_:
            setattr(arr[l], f, None if f == null_field else FAKE)
    w = dflash_weights(w_fuse=FAKE, embed=FAKE, final_norm=FAKE, lm_head=FAKE, rope_cos=FAKE, rope_sin=FAKE,
                       rope_rows=1024, layers=ctypes.cast(arr, ctypes.POINTER(dflash_layer_weights)))
    w._keep = arr
    return w


def _kv():
    return dflash_kv(k=FAKE, v=FAKE, len=FAKE, status=FAKE)


def test_inject_host_errors():
    L = _lib()
    c, w, kv = _cfg(), _weights(), _kv()
    ws_need = L.dflash_workspace_bytes(ctypes.byref(c), 1, 8)
    call = lambda **k: L.dflash_inject_kv(ctypes.byref(k.get("c", c)), ctypes.byref(k.get("w", w)),
                                          ctypes.byref(k.get("kv", kv)), k.get("batch", 1), k.get("feat", FAKE),
                                          k.get("rows", 8), k.get("n_new", FAKE), k.get("ws", FAKE),
                                          k.get("wsb", ws_need), None)
    assert call(batch=0) == DFLASH_EINVAL
    assert call(batch=2) == DFLASH_EINVAL
    assert call(rows=0) == DFLASH_EINVAL
    assert call(feat=None) == DFLASH_EINVAL
    assert call(n_new=None) == DFLASH_EINVAL
    assert call(kv=dflash_kv(k=FAKE, v=FAKE, len=None, status=FAKE)) == DFLASH_EINVAL
    assert call(w=_weights(null_field="wk")) == DFLASH_EINVAL
    assert call(ws=None) == DFLASH_EWORKSPACE
    assert call(wsb=ws_need - 1) == DFLASH_EWORKSPACE
    assert call(rows=9) == DFLASH_EWORKSPACE        # workspace sized for 8 rows
    assert call(c=_cfg(head_dim=32)) == DFLASH_EUNSUPPORTED
    small = _weights()
    small.rope_rows = 10
    assert call(w=small) == DFLASH_EINVAL


def test_draft_host_errors():
    L = _lib()
    c, w, kv = _cfg(), _weights(), _kv()
    ws_need = L.dflash_workspace_bytes(ctypes.byref(c), 1, 0)
    call = lambda **k: L.dflash_draft_block(ctypes.byref(k.get("c", c)), ctypes.byref(w), ctypes.byref(kv),
                                            k.get("batch", 1), k.get("gamma", 8), k.get("anchor", FAKE),
                                            k.get("draft", FAKE), None, None, k.get("ws", FAKE),
                                            k.get("wsb", ws_need), None)
    assert call(gamma=1) == DFLASH_EINVAL
    assert call(gamma=9) == DFLASH_EINVAL           # > gamma_max
    assert call(batch=0) == DFLASH_EINVAL
    assert call(anchor=None) == DFLASH_EINVAL
    assert call(draft=None) == DFLASH_EINVAL
    assert call(wsb=ws_need - 256) == DFLASH_EWORKSPACE
    assert call(c=_cfg(mask_token_id=5000)) == DFLASH_EINVAL
    assert call(c=_cfg(n_q_heads=3)) == DFLASH_EUNSUPPORTED


def test_block_loss_host_errors():
    L = _lib()
    c, w, kv = _cfg(), _weights(), _kv()
    ws_need = L.dflash_workspace_bytes(ctypes.byref(c), 1, 0)
    call = lambda **k: L.dflash_block_loss(ctypes.byref(k.get("c", c)), ctypes.byref(k.get("w", w)), ctypes.byref(kv),
                                           k.get("batch", 1), k.get("gamma", 8), k.get("anchor", FAKE),
                                           k.get("labels", FAKE), k.get("loss", FAKE), None, None, None,
                                           k.get("ws", FAKE), k.get("wsb", ws_need), None)
    assert call(gamma=1) == DFLASH_EINVAL
    assert call(gamma=9) == DFLASH_EINVAL           # > gamma_max
    assert call(batch=0) == DFLASH_EINVAL
    assert call(anchor=None) == DFLASH_EINVAL
    assert call(labels=None) == DFLASH_EINVAL
    assert call(loss=None) == DFLASH_EINVAL
    assert call(w=_weights(null_field="w_down")) == DFLASH_EINVAL
    assert call(ws=None) == DFLASH_EWORKSPACE
    assert call(wsb=ws_need - 256) == DFLASH_EWORKSPACE
    assert call(c=_cfg(head_dim=32)) == DFLASH_EUNSUPPORTED


def test_input_fusion_host_errors():
    L = _lib()
    c, w, kv = _cfg(), _weights(), _kv()
    ws_need = L.dflash_workspace_bytes(ctypes.byref(c), 1, 8)
    call = lambda **k: L.dflash_inject_kv_input_fusion(
        ctypes.byref(k.get("c", c)), ctypes.byref(k.get("w", w)), ctypes.byref(k.get("kv", kv)), k.get("batch", 1),
        k.get("feat", FAKE), k.get("rows", 8), k.get("n_new", FAKE), k.get("ws", FAKE), k.get("wsb", ws_need), None)
    assert call(batch=0) == DFLASH_EINVAL
    assert call(batch=2) == DFLASH_EINVAL
    assert call(rows=0) == DFLASH_EINVAL
    assert call(rows=9) == DFLASH_EINVAL            # more rows than gamma_max
    assert call(feat=None) == DFLASH_EINVAL
    assert call(n_new=None) == DFLASH_EINVAL
    assert call(kv=dflash_kv(k=FAKE, v=FAKE, len=None, status=FAKE)) == DFLASH_EINVAL
    assert call(w=_weights(null_field="wq")) == DFLASH_EINVAL
    assert call(ws=None) == DFLASH_EWORKSPACE
    assert call(wsb=ws_need - 1) == DFLASH_EWORKSPACE
    assert call(c=_cfg(head_dim=32)) == DFLASH_EUNSUPPORTED


def test_verify_host_errors():
    L = _lib()
    assert L.dflash_verify(0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == DFLASH_EINVAL
    assert L.dflash_verify(1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == DFLASH_EINVAL
    assert L.dflash_verify(1, 1025, FAKE, FAKE, FAKE, FAKE, FAKE, None) == DFLASH_EINVAL
    assert L.dflash_verify(1, 4, None, FAKE, FAKE, FAKE, FAKE, None) == DFLASH_EINVAL
    assert L.dflash_verify(1, 4, FAKE, FAKE, FAKE, None, FAKE, None) == DFLASH_EINVAL


def test_status_strings():
    L = _lib()
    for code in (0, -1, -2, -3, -4):
        assert L.dflash_status_str(code).startswith(b"DFLASH_")
    assert L.dflash_status_str(99) == b"unknown dflash status"


def test_traced_variants_validate_like_the_plain_calls():
    L = _lib()
    c, w, kv = _cfg(), _weights(), _kv()
    ws_need = L.dflash_workspace_bytes(ctypes.byref(c), 1, 8)
    bad = dflash_trace(events=None, capacity=-1, count=0, names=None)
    good = dflash_trace(events=None, capacity=0, count=0, names=None)
    assert L.dflash_inject_kv_traced(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), 1, FAKE, 8, FAKE, FAKE,
                                     ws_need, None, ctypes.byref(bad)) == DFLASH_EINVAL
    assert L.dflash_inject_kv_traced(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), 0, FAKE, 8, FAKE, FAKE,
                                     ws_need, None, ctypes.byref(good)) == DFLASH_EINVAL
    assert L.dflash_draft_block_traced(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), 1, 1, FAKE, FAKE,
                                       None, None, FAKE, ws_need, None, ctypes.byref(good)) == DFLASH_EINVAL


def test_binding_checks_tensor_arguments_before_calling_the_library():
    # the binding passes raw pointers, so it must reject what the C side cannot see
    import types
    import torch
    import block_diffusion_drafter_states_amd as dfl
    cfg = synth.get_config("C1")
    model = types.SimpleNamespace(cfg=cfg, storage_dtype=torch.float32)
    cpu_feat = torch.zeros((1, 4, cfg.n_feat, cfg.hidden), dtype=torch.float32)
    cpu_i32 = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(TypeError, match="device tensor"):
        dfl.inject_kv(model, None, cpu_feat, cpu_i32, None)
    with pytest.raises(TypeError, match="device tensor"):
        dfl.draft_block(model, None, 8, cpu_i32, torch.zeros((1, 7), dtype=torch.int32), None)
    with pytest.raises(TypeError, match="device tensor"):
        dfl.verify(torch.zeros((1, 7), dtype=torch.int32), torch.zeros((1, 8), dtype=torch.int32),
                   cpu_i32, torch.zeros((1, 8), dtype=torch.int32), cpu_i32)


def test_head_composite_reading():
    """The argmax-head composite the GPU checks compare with (rho(x * w) . W^T times the final
    norm's row factor) against the oracle's own final stage (rho(RMSNorm(x; w)) . W^T): equal
    to fp64 noise without rounding, within one bf16 rounding of the input with it, and the
    same argmax wherever the top two logits are clearly apart."""
    import numpy as np
    import gpu_support as G
    import oracle.dflash as O
    for dtype in ("f32", "bf16"):
        cfg = synth.Config(f"head_{dtype}", dtype, hidden=256, n_q=2, n_kv=1, head_dim=128 if dtype == "bf16" else 64,
                           inter=512, n_layers=1, n_feat=2, vocab=700, gamma=8, ctx=16, batch=1, index=95)
        om = O.DraftModel(cfg, gen.weights(cfg))
        x = 3.0 * np.random.default_rng(7).standard_normal((2, cfg.gamma, cfg.hidden))
        got = G.oracle_head(om)(x)
        ref = O.linear(om.num.rho(O.rms_norm(x[:, 1:], om.final_norm, cfg.eps)), om.lm_head)
        err = np.abs(got - ref).max() / np.abs(ref).max()
        if dtype == "f32":      # the oracle computes in fp64 and rho rounds nothing here
            assert err < 1e-12
        else:
            assert 1e-6 < err < 1e-2
            srt = np.sort(ref, axis=-1)
            clear = srt[..., -1] - srt[..., -2] > 20 * np.abs(got - ref).max()
            assert clear.sum() > 0
            assert (np.argmax(got, -1) == np.argmax(ref, -1))[clear].all()


def test_draft_check_flags_wrong_ids():
    """The GPU draft check itself: exact ids where the oracle's top-2 gap is at least 1e-2,
    self-consistent argmax, near-optimal choice elsewhere, per-row relative errors; mistakes
    are planted in the reference-side arrays on the CPU."""
    import numpy as np
    import gpu_support as G
    cfg = type("C", (), {"dtype": "bf16"})()
    rng = np.random.default_rng(5)
    zr = rng.standard_normal((3, 7, 50))
    z = zr + 1e-3 * rng.standard_normal(zr.shape)
    d = np.argmax(z, axis=-1)
    x = rng.standard_normal((3, 8, 4))
    good = G.check_draft(cfg, (d, x, z), (np.argmax(zr, -1), x, zr))
    G.assert_draft(cfg, good)
    bad_d = d.copy()
    bad_d[1, 2] = np.argmin(z[1, 2])
    m = G.check_draft(cfg, (bad_d, x, z), (np.argmax(zr, -1), x, zr))
    assert m["argmax_self_mismatch"] == 1 and m["not_near_optimal"] == 1
    with pytest.raises(AssertionError):
        G.assert_draft(cfg, m)
    # ids that are the argmax of the returned logits, but one logit is far off the
    # reference: the margin widens so no id is sure, and the logit bound fails
    z2 = z.copy()
    z2[0, 0, np.argmin(zr[0, 0])] = zr[0, 0].max() + 5.0
    m = G.check_draft(cfg, (np.argmax(z2, -1), x, z2), (np.argmax(zr, -1), x, zr))
    assert m["argmax_self_mismatch"] == 0 and m["logits_rel"] > G.tol(cfg)
    with pytest.raises(AssertionError):
        G.assert_draft(cfg, m)
    # one hidden row off by 20%: the whole-tensor error stays small, the per-row bound fails
    xb = x.copy()
    xb[2, 3] *= 1.2
    m = G.check_draft(cfg, (d, x, z), (np.argmax(zr, -1), xb, zr))
    assert m["hidden_rel"] < G.tol(cfg) * 10 and m["hidden_row_max"] > G.tol(cfg)
    with pytest.raises(AssertionError):
        G.assert_draft(cfg, m)
    # a row with a 5e-2 top-2 gap whose id differs is a strict mismatch, counted by band
    zs = zr.copy()
    zs[0, 1] = np.sort(zs[0, 1])        # ascending: the last id is the maximum
    zs[0, 1, -2] = zs[0, 1, -1] - 5e-2
    ds = np.argmax(zs, -1)
    ds[0, 1] = zs.shape[-1] - 2
    m = G.check_draft(cfg, (ds, x, zs), (np.argmax(zs, -1), x, zs))
    assert m["strict_mismatch"] == 1 and m["wide_mismatch"] == 1 and m["band_exempt_differ"] == 0
    with pytest.raises(AssertionError):
        G.assert_draft(cfg, m)
    # the LM-head stage on the GPU's own hidden rows: a differing id at gap >= 1e-2 fails
    # even where the end-to-end comparison would allow it
    m = G.check_draft(cfg, (d, x, z), (np.argmax(zr, -1), x, zr), head=lambda h: z)
    assert m["head_strict_mismatch"] == 0 and m["head_checked"] > 0
    G.assert_draft(cfg, m)
    zh = z.copy()
    zh[2, 4] = np.sort(zh[2, 4])
    zh[2, 4, 0] = zh[2, 4, -1] + 1.0        # the head's argmax is now id 0 with a clear gap
    m = G.check_draft(cfg, (d, x, z), (np.argmax(zr, -1), x, zr), head=lambda h: zh)
    assert m["head_strict_mismatch"] == (0 if d[2, 4] == 0 else 1)
    if d[2, 4] != 0:
        with pytest.raises(AssertionError):
            G.assert_draft(cfg, m)


def test_probe_library_exports_and_rejects_bad_arguments():
    """libdflash_probe.so (the benchmark's measured ceilings, `bench.py --probes`) exports the
    two HBM-read and the two MFMA probes, and each returns -1 for invalid arguments before any launch."""
    path = os.path.join(os.path.dirname(_abi.LIB_PATH), "libdflash_probe.so")
    if not os.path.exists(path):
        pytest.skip("libdflash_probe.so not built (run __graft_entry__.build())")
    P = ctypes.CDLL(path)
    out = os.popen(f"nm -D --defined-only {path}").read()
    names = sorted(re.findall(r"\bT (dflash_probe_[a-z0-9_]+)\b", out))
    assert names == ["dflash_probe_mfma", "dflash_probe_mfma32", "dflash_probe_read", "dflash_probe_read_nt"]
    P.dflash_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    P.dflash_probe_read_nt.argtypes = P.dflash_probe_read.argtypes
    P.dflash_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.dflash_probe_mfma32.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert P.dflash_probe_read(None, 16, 0, None, 1, None) == -1
    assert P.dflash_probe_read(None, 15, 0, None, 1, None) == -1
    assert P.dflash_probe_read_nt(None, 16, 0, None, 1, None) == -1
    assert P.dflash_probe_read_nt(None, 16, 0, None, 0, None) == -1
    assert P.dflash_probe_mfma(1, 1, None, None) == -1
    assert P.dflash_probe_mfma32(0, 1, None, None) == -1


def test_advance_len_host_errors():
    """The capacity comes from the configuration (the one the cache was sized with), so the
    call validates the configuration and the batch against it."""
    L = _lib()
    c, kv = _cfg(), _kv()
    call = lambda **k: L.dflash_advance_len(ctypes.byref(k.get("c", c)), ctypes.byref(k.get("kv", kv)),
                                            k.get("batch", 1), k.get("n", FAKE), None)
    assert call(batch=0) == DFLASH_EINVAL
    assert call(batch=2) == DFLASH_EINVAL            # max_batch 1
    assert call(n=None) == DFLASH_EINVAL
    assert call(kv=dflash_kv(k=FAKE, v=FAKE, len=None, status=FAKE)) == DFLASH_EINVAL
    assert call(c=_cfg(kv_capacity=100)) == DFLASH_EUNSUPPORTED
    assert L.dflash_advance_len(None, ctypes.byref(kv), 1, FAKE, None) == DFLASH_EINVAL


def test_noalloc_rejects_calls_beyond_the_fixed_scratch():
    """dflash_draft_block_noalloc validates like dflash_draft_block and refuses, before any
    device call, a call whose workspace exceeds the library's fixed per-GPU array."""
    L = _lib()
    assert L.dflash_noalloc_scratch_bytes() == 64 << 20
    c5 = synth.get_config("C5")
    big = dflash_config(hidden=c5.hidden, n_q_heads=c5.n_q, n_kv_heads=c5.n_kv, head_dim=c5.head_dim,
                        inter=c5.inter, n_layers=c5.n_layers, n_feat=c5.n_feat, vocab=c5.vocab, gamma_max=16,
                        mask_token_id=c5.mask_id, max_batch=12, kv_capacity=32832, rms_eps=1e-6, dtype=1)
    assert L.dflash_workspace_bytes(ctypes.byref(big), 12, 0) > L.dflash_noalloc_scratch_bytes()
    w = _weights(c5.n_layers)
    w.rope_rows = 32832 + 16
    call = lambda **k: L.dflash_draft_block_noalloc(ctypes.byref(k.get("c", big)), ctypes.byref(k.get("w", w)),
                                                    ctypes.byref(_kv()), k.get("batch", 12), k.get("gamma", 16),
                                                    FAKE, k.get("draft", FAKE), None, None, None)
    assert call() == _abi.DFLASH_ESCRATCH
    assert b"DFLASH_ESCRATCH" in L.dflash_status_str(_abi.DFLASH_ESCRATCH)
    assert call(batch=13) == DFLASH_EINVAL
    assert call(gamma=17) == DFLASH_EINVAL
    assert call(draft=None) == DFLASH_EINVAL
    assert call(w=_weights(c5.n_layers, null_field="wo")) == DFLASH_EINVAL
