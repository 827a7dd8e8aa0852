"""DFlash drafting + verification cycle on AMD gfx950 (MI355X).

Thin Python binding of ``libdflash.so`` (C ABI in ``include/dflash.h``).  The
three calls carry the names of the C entry points:

    inject_kv(model, cache, feat, n_new, ws)         -> dflash_inject_kv
    draft_block(model, cache, gamma, anchor, draft)  -> dflash_draft_block
    verify(draft, target, accept_len, committed, next_anchor) -> dflash_verify

PyTorch only provides device memory and the stream; every step of the cycle
runs in the HIP kernels.  ``Model``, ``Cache`` and ``Workspace`` hold the
device tensors and build the C structs that point into them.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import _abi
from ._abi import (dflash_config, dflash_kv, dflash_layer_weights, dflash_weights, check, lib,  # noqa: F401
                   DFlashError, STATUS_BAD_COUNT, STATUS_BAD_TOKEN, STATUS_KV_OVERFLOW)

LAYER_FIELDS = ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down")


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, device):
    """Storage array (bf16 bit patterns as uint16, or fp32) -> device tensor of the storage dtype."""
    torch = _torch()
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    if arr.dtype == np.float32:
        return torch.from_numpy(arr).to(device)
    raise TypeError(f"unsupported storage dtype {arr.dtype}")


def to_storage(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> host storage array (uint16 bit patterns or fp32)."""
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def rope_table(head_dim: int, theta: float, rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """Host-built RoPE table [rows][D/2]: cos and sin of p * theta^(-2i/D), angles in fp64,
    rounded once to fp32 (no device-side sin/cos or range reduction)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = np.power(float(theta), -2.0 * i / head_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _stream_ptr(stream) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Model:
    """Drafter weights resident on the device plus the C-side config/weights structs.

    ``cfg`` is a ``synth.Config``-like object (fields hidden, n_q, n_kv, head_dim,
    inter, n_layers, n_feat, vocab, mask_id, eps, rope_theta, dtype); ``W`` maps
    names to storage arrays (``lm_head`` may be the same object as ``embed``).
    """

    def __init__(self, cfg, W: Dict[str, object], device="cuda", max_batch: int = 1,
                 kv_capacity: int = 64, gamma_max: Optional[int] = None, share_from: Optional["Model"] = None):
        """``share_from``: a model whose embedding and LM head tensors this one uses (a
        verifying target and its drafter share them); ``W['w_fuse']`` may then be absent."""
        self.cfg = cfg
        self.device = device
        gmax = gamma_max if gamma_max is not None else cfg.gamma_max
        self.c = dflash_config(hidden=cfg.hidden, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                               head_dim=cfg.head_dim, inter=cfg.inter, n_layers=cfg.n_layers,
                               n_feat=cfg.n_feat, vocab=cfg.vocab, gamma_max=gmax,
                               mask_token_id=cfg.mask_id, max_batch=max_batch, kv_capacity=kv_capacity,
                               rms_eps=cfg.eps, dtype=_abi.DFLASH_BF16 if cfg.dtype == "bf16" else _abi.DFLASH_F32)
        up = lambda a: to_device(a, device)
        self.t = {"final_norm": up(W["final_norm"])}
        self.t["w_fuse"] = up(W["w_fuse"]) if W.get("w_fuse") is not None else None
        if share_from is not None:
            self.t["embed"], self.t["lm_head"] = share_from.t["embed"], share_from.t["lm_head"]
        else:
            self.t["embed"] = up(W["embed"])
            self.t["lm_head"] = self.t["embed"] if W["lm_head"] is W["embed"] else up(W["lm_head"])
        cos, sin = rope_table(cfg.head_dim, cfg.rope_theta, kv_capacity + gmax)
        self.t["rope_cos"] = _torch().from_numpy(cos).to(device)
        self.t["rope_sin"] = _torch().from_numpy(sin).to(device)
        self.layers = [{k: up(v) for k, v in lw.items()} for lw in W["layers"]]
        arr = (dflash_layer_weights * cfg.n_layers)()
        for l, lw in enumerate(self.layers):
            for f in LAYER_FIELDS:
                setattr(arr[l], f, lw[f].data_ptr())
        self._layer_arr = arr
        fuse_ptr = self.t["w_fuse"].data_ptr() if self.t["w_fuse"] is not None else None
        self.w = dflash_weights(w_fuse=fuse_ptr, embed=self.t["embed"].data_ptr(),
                                final_norm=self.t["final_norm"].data_ptr(), lm_head=self.t["lm_head"].data_ptr(),
                                rope_cos=self.t["rope_cos"].data_ptr(), rope_sin=self.t["rope_sin"].data_ptr(),
                                rope_rows=kv_capacity + gmax,
                                layers=ctypes.cast(arr, ctypes.POINTER(dflash_layer_weights)))

    @property
    def storage_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32


class Cache:
    """Draft KV cache: K [L][B][n_kv][cap][D]; V in blocks of 32 positions, each transposed,
    [L][B][n_kv][cap/32][D][32]; len[B], status."""

    def __init__(self, model: Model):
        torch = _torch()
        c = model.c
        L, B, nkv, cap, D = c.n_layers, c.max_batch, c.n_kv_heads, c.kv_capacity, c.head_dim
        dt = model.storage_dtype
        self.k = torch.zeros((L, B, nkv, cap, D), dtype=dt, device=model.device)
        self.v = torch.zeros((L, B, nkv, cap // 32, D, 32), dtype=dt, device=model.device)
        self.len = torch.zeros(B, dtype=torch.int32, device=model.device)
        self.status = torch.zeros(1, dtype=torch.int32, device=model.device)
        self.s = dflash_kv(k=self.k.data_ptr(), v=self.v.data_ptr(), len=self.len.data_ptr(),
                           status=self.status.data_ptr())

    def set_context(self, K: np.ndarray, V: np.ndarray, lengths: Sequence[int]) -> None:
        """Upload a context cache given as storage arrays K, V [L][B][n_kv][C][D] (C <= cap)."""
        torch = _torch()
        C = K.shape[3]
        B = K.shape[1]
        self.k.zero_()
        self.v.zero_()
        self.k[:, :B, :, :C, :] = to_device(K, self.k.device)
        nb = (C + 31) // 32                                 # 32-position blocks, each transposed
        vd = to_device(V, self.v.device)
        if nb * 32 != C:
            vd = torch.cat([vd, vd.new_zeros(vd.shape[:3] + (nb * 32 - C, vd.shape[4]))], dim=3)
        self.v[:, :B, :, :nb] = vd.reshape(vd.shape[:3] + (nb, 32, vd.shape[4])).transpose(-1, -2)
        self.len[:B] = torch.as_tensor(np.asarray(lengths, dtype=np.int32), device=self.len.device)

    def read_k(self) -> np.ndarray:
        return to_storage(self.k)

    def read_v(self) -> np.ndarray:
        """V as [L][B][n_kv][cap][D] storage (the 32-position blocks un-transposed)."""
        v = self.v.transpose(-1, -2).contiguous()
        return to_storage(v.reshape(v.shape[:3] + (-1, v.shape[-1])))


class Workspace:
    def __init__(self, model: Model, batch: int, max_rows_per_seq: int):
        torch = _torch()
        self.nbytes = workspace_bytes(model, batch, max_rows_per_seq)
        if self.nbytes == 0:
            raise DFlashError(_abi.DFLASH_EUNSUPPORTED, "dflash_workspace_bytes")
        # scratch: every call writes what it reads, nothing survives a call
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=model.device)

    def ptr(self) -> int:
        return self.buf.data_ptr()


# ----------------------------------------------------------------------------- entry points

def _need(t, name: str, dtype, shape: Sequence[Optional[int]]) -> None:
    """The C ABI takes raw pointers: check what it cannot (device, dtype, layout, shape)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if t.dim() != len(shape) or any(s is not None and s != n for s, n in zip(shape, t.shape)):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def workspace_bytes(model: Model, batch: int, max_rows_per_seq: int) -> int:
    return int(lib().dflash_workspace_bytes(ctypes.byref(model.c), batch, max_rows_per_seq))


def inject_kv(model: Model, cache: Cache, feat, n_new, ws: Workspace, batch: Optional[int] = None,
              stream=None) -> None:
    """feat: device tensor [batch][rows][F][H] (storage dtype); n_new: device int32 [batch]."""
    torch = _torch()
    batch = feat.shape[0] if batch is None else batch
    rows = feat.shape[1]
    _need(feat, "feat", model.storage_dtype, (None, rows, model.cfg.n_feat, model.cfg.hidden))
    if batch > feat.shape[0]:
        raise ValueError(f"feat holds {feat.shape[0]} sequences, batch is {batch}")
    _need(n_new, "n_new", torch.int32, (None,))
    if n_new.shape[0] < batch:
        raise ValueError(f"n_new holds {n_new.shape[0]} entries, batch is {batch}")
    check(lib().dflash_inject_kv(ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s), batch,
                                 feat.data_ptr(), rows, n_new.data_ptr(), ws.ptr(), ws.nbytes,
                                 _stream_ptr(stream)), "dflash_inject_kv")


def inject_kv_input_fusion(model: Model, cache: Cache, feat, n_new, ws: Workspace, batch: Optional[int] = None,
                           stream=None) -> None:
    """Input-fusion conditioning (cost comparison with inject_kv): feat [batch][rows][F][H] storage,
    rows <= gamma_max; every draft layer runs over the fused rows and keeps their K/V; len += n_new."""
    torch = _torch()
    batch = feat.shape[0] if batch is None else batch
    rows = feat.shape[1]
    _need(feat, "feat", model.storage_dtype, (None, rows, model.cfg.n_feat, model.cfg.hidden))
    if batch > feat.shape[0]:
        raise ValueError(f"feat holds {feat.shape[0]} sequences, batch is {batch}")
    _need(n_new, "n_new", torch.int32, (None,))
    if n_new.shape[0] < batch:
        raise ValueError(f"n_new holds {n_new.shape[0]} entries, batch is {batch}")
    check(lib().dflash_inject_kv_input_fusion(ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s),
                                              batch, feat.data_ptr(), rows, n_new.data_ptr(), ws.ptr(), ws.nbytes,
                                              _stream_ptr(stream)), "dflash_inject_kv_input_fusion")


def draft_block(model: Model, cache: Cache, gamma: int, anchor, draft, ws: Workspace, dbg_hidden=None,
                dbg_logits=None, stream=None) -> None:
    """anchor: device int32 [batch]; draft: device int32 [batch][gamma-1] (output)."""
    torch = _torch()
    batch = anchor.shape[0]
    _need(anchor, "anchor", torch.int32, (batch,))
    _need(draft, "draft", torch.int32, (batch, gamma - 1))
    if dbg_hidden is not None:
        _need(dbg_hidden, "dbg_hidden", torch.float32, (batch, gamma, model.cfg.hidden))
    if dbg_logits is not None:
        _need(dbg_logits, "dbg_logits", torch.float32, (batch, gamma - 1, model.cfg.vocab))
    check(lib().dflash_draft_block(ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s), batch,
                                   gamma, anchor.data_ptr(), draft.data_ptr(),
                                   None if dbg_hidden is None else dbg_hidden.data_ptr(),
                                   None if dbg_logits is None else dbg_logits.data_ptr(),
                                   ws.ptr(), ws.nbytes, _stream_ptr(stream)), "dflash_draft_block")


def draft_block_noalloc(model: Model, cache: Cache, gamma: int, anchor, draft, dbg_hidden=None, dbg_logits=None,
                        stream=None) -> None:
    """draft_block without a workspace: the library's fixed per-GPU scratch is used instead
    (dflash_draft_block_noalloc; calls that may overlap on one GPU race)."""
    torch = _torch()
    batch = anchor.shape[0]
    _need(anchor, "anchor", torch.int32, (batch,))
    _need(draft, "draft", torch.int32, (batch, gamma - 1))
    if dbg_hidden is not None:
        _need(dbg_hidden, "dbg_hidden", torch.float32, (batch, gamma, model.cfg.hidden))
    if dbg_logits is not None:
        _need(dbg_logits, "dbg_logits", torch.float32, (batch, gamma - 1, model.cfg.vocab))
    check(lib().dflash_draft_block_noalloc(ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s),
                                           batch, gamma, anchor.data_ptr(), draft.data_ptr(),
                                           None if dbg_hidden is None else dbg_hidden.data_ptr(),
                                           None if dbg_logits is None else dbg_logits.data_ptr(),
                                           _stream_ptr(stream)), "dflash_draft_block_noalloc")


def block_loss(model: Model, cache: Cache, gamma: int, anchor, labels, loss, ws: Workspace, row_loss=None,
               dbg_logits=None, stream=None, dlogits=None) -> None:
    """The drafter's weighted block cross-entropy: anchor int32 [B], labels int32 [B][gamma-1]
    -> loss fp32 [1] (weights exp(-(j-1)/gamma) on mask row j), row_loss fp32 [B][gamma-1],
    dlogits fp32 [B][gamma-1][V] (gradient of the loss w.r.t. the mask rows' logits)."""
    torch = _torch()
    batch = anchor.shape[0]
    _need(anchor, "anchor", torch.int32, (batch,))
    _need(labels, "labels", torch.int32, (batch, gamma - 1))
    _need(loss, "loss", torch.float32, (1,))
    if row_loss is not None:
        _need(row_loss, "row_loss", torch.float32, (batch, gamma - 1))
    if dbg_logits is not None:
        _need(dbg_logits, "dbg_logits", torch.float32, (batch, gamma - 1, model.cfg.vocab))
    if dlogits is not None:
        _need(dlogits, "dlogits", torch.float32, (batch, gamma - 1, model.cfg.vocab))
    check(lib().dflash_block_loss(ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s), batch,
                                  gamma, anchor.data_ptr(), labels.data_ptr(), loss.data_ptr(),
                                  None if row_loss is None else row_loss.data_ptr(),
                                  None if dlogits is None else dlogits.data_ptr(),
                                  None if dbg_logits is None else dbg_logits.data_ptr(),
                                  ws.ptr(), ws.nbytes, _stream_ptr(stream)), "dflash_block_loss")


def verify(draft, target, accept_len, committed, next_anchor, stream=None) -> None:
    """draft int32 [B][gamma-1], target int32 [B][gamma] -> accept_len [B], committed [B][gamma], next_anchor [B]."""
    torch = _torch()
    _need(target, "target", torch.int32, (None, None))
    B, gamma = target.shape
    _need(draft, "draft", torch.int32, (B, gamma - 1))
    _need(accept_len, "accept_len", torch.int32, (B,))
    _need(committed, "committed", torch.int32, (B, gamma))
    _need(next_anchor, "next_anchor", torch.int32, (B,))
    check(lib().dflash_verify(B, gamma, draft.data_ptr(), target.data_ptr(), accept_len.data_ptr(),
                              committed.data_ptr(), next_anchor.data_ptr(), _stream_ptr(stream)), "dflash_verify")


def target_forward(model: Model, cache: Cache, tokens, y, ws: Workspace, feat=None, taps: Sequence[int] = (),
                   dbg_logits=None, stream=None) -> None:
    """A verifying target's causal forward over tokens int32 [B][rows] at positions len..: writes
    the rows' K/V, y int32 [B][rows] (argmax), feat storage [B][rows][len(taps)][H] (hidden states
    after the 1-based decoder layers in taps), dbg_logits fp32 [B][rows][V]; len unchanged."""
    torch = _torch()
    _need(tokens, "tokens", torch.int32, (None, None))
    B, rows = tokens.shape
    _need(y, "y", torch.int32, (B, rows))
    taps = [int(t) for t in taps]
    if taps:
        _need(feat, "feat", model.storage_dtype, (B, rows, len(taps), model.cfg.hidden))
    if dbg_logits is not None:
        _need(dbg_logits, "dbg_logits", torch.float32, (B, rows, model.cfg.vocab))
    tap_arr = (ctypes.c_int32 * max(1, len(taps)))(*taps)
    check(lib().dflash_target_forward(ctypes.byref(model.c), ctypes.byref(model.w), ctypes.byref(cache.s), B, rows,
                                      tokens.data_ptr(), y.data_ptr(), None if not taps else feat.data_ptr(),
                                      tap_arr if taps else None, len(taps),
                                      None if dbg_logits is None else dbg_logits.data_ptr(), ws.ptr(), ws.nbytes,
                                      _stream_ptr(stream)), "dflash_target_forward")


def advance_len(model: Model, cache: Cache, n, batch: Optional[int] = None, stream=None) -> None:
    """len[b] += n[b] (n device int32 [batch], e.g. verify's accept_len)."""
    torch = _torch()
    _need(n, "n", torch.int32, (None,))
    batch = n.shape[0] if batch is None else batch
    check(lib().dflash_advance_len(ctypes.byref(model.c), ctypes.byref(cache.s), batch, n.data_ptr(),
                                   _stream_ptr(stream)), "dflash_advance_len")


def choose_gamma(tau: Sequence[int], gamma_used: Sequence[int], cost_us: Sequence[float], gamma_min: int = 2,
                 gamma_max: int = 16, prior_p: float = 0.8, prior_weight: float = 4.0) -> Tuple[int, float]:
    """Block size for the next cycle from recent (accept length, block size) pairs and a table
    cost_us[g] (g = 0..gamma_max, <= 0: not a candidate) of measured cycle times; returns
    (gamma, estimated per-position acceptance).  Host-only (dflash_choose_gamma)."""
    n = len(tau)
    if len(gamma_used) != n or len(cost_us) < gamma_max + 1:
        raise ValueError("tau / gamma_used lengths differ or cost_us is shorter than gamma_max + 1")
    t = (ctypes.c_int32 * max(1, n))(*tau)
    g = (ctypes.c_int32 * max(1, n))(*gamma_used)
    c = (ctypes.c_float * len(cost_us))(*cost_us)
    out_g, out_p = ctypes.c_int32(0), ctypes.c_double(0.0)
    check(lib().dflash_choose_gamma(t, g, n, c, gamma_min, gamma_max, prior_p, prior_weight, ctypes.byref(out_g),
                                    ctypes.byref(out_p)), "dflash_choose_gamma")
    return int(out_g.value), float(out_p.value)


def status_str(code: int) -> str:
    return lib().dflash_status_str(code).decode()
