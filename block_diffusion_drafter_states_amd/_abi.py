"""ctypes mirror of include/dflash.h and the loader of libdflash.so.

Argument marshalling only: every step of the cycle runs in the HIP library.
Importing this module does not touch a GPU; calling ``lib()`` loads the shared
library and raises if it has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB_PATH selects another build of the same sources (the host-sanitized one of the
# host-only tests); by default the in-tree library.
LIB_PATH = os.environ.get("DFLASH_LIB_PATH") or os.path.join(HERE, "libdflash.so")

DFLASH_OK = 0
DFLASH_EINVAL = -1
DFLASH_EUNSUPPORTED = -2
DFLASH_EWORKSPACE = -3
DFLASH_ELAUNCH = -4
DFLASH_ESCRATCH = -5

DFLASH_F32 = 0
DFLASH_BF16 = 1

STATUS_KV_OVERFLOW = 1
STATUS_BAD_TOKEN = 2
STATUS_BAD_COUNT = 4

EXPORTED = ("dflash_workspace_bytes", "dflash_inject_kv", "dflash_draft_block", "dflash_verify",
            "dflash_inject_kv_traced", "dflash_draft_block_traced", "dflash_target_forward", "dflash_advance_len",
            "dflash_choose_gamma", "dflash_block_loss", "dflash_inject_kv_input_fusion", "dflash_audit_workspace",
            "dflash_draft_block_noalloc", "dflash_noalloc_scratch_bytes", "dflash_status_str")


class dflash_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_feat", ctypes.c_int32), ("vocab", ctypes.c_int32), ("gamma_max", ctypes.c_int32),
                ("mask_token_id", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("kv_capacity", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class dflash_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down")]


class dflash_weights(ctypes.Structure):
    _fields_ = [("w_fuse", ctypes.c_void_p), ("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p),
                ("rope_rows", ctypes.c_int32), ("layers", ctypes.POINTER(dflash_layer_weights))]


class dflash_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


class dflash_trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32), ("names", ctypes.POINTER(ctypes.c_char_p))]


_LIB = None


def lib(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdflash.so (once).  Raises RuntimeError when it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m block_diffusion_drafter_states_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    L.dflash_workspace_bytes.restype = ctypes.c_size_t
    L.dflash_workspace_bytes.argtypes = [P(dflash_config), ctypes.c_int32, ctypes.c_int32]
    L.dflash_inject_kv.restype = ctypes.c_int
    L.dflash_inject_kv.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    L.dflash_draft_block.restype = ctypes.c_int
    L.dflash_draft_block.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.dflash_verify.restype = ctypes.c_int
    L.dflash_verify.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.dflash_inject_kv_traced.restype = ctypes.c_int
    L.dflash_inject_kv_traced.argtypes = L.dflash_inject_kv.argtypes + [P(dflash_trace)]
    L.dflash_draft_block_traced.restype = ctypes.c_int
    L.dflash_draft_block_traced.argtypes = L.dflash_draft_block.argtypes + [P(dflash_trace)]
    L.dflash_target_forward.restype = ctypes.c_int
    L.dflash_target_forward.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
    L.dflash_advance_len.restype = ctypes.c_int
    L.dflash_advance_len.argtypes = [P(dflash_config), P(dflash_kv), ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.dflash_draft_block_noalloc.restype = ctypes.c_int
    L.dflash_draft_block_noalloc.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]
    L.dflash_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.dflash_noalloc_scratch_bytes.argtypes = []
    L.dflash_audit_workspace.restype = ctypes.c_int
    L.dflash_audit_workspace.argtypes = [P(dflash_config), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         P(ctypes.c_int32), P(ctypes.c_int32), P(ctypes.c_int32)]
    L.dflash_choose_gamma.restype = ctypes.c_int
    L.dflash_choose_gamma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
    L.dflash_inject_kv_input_fusion.restype = ctypes.c_int
    L.dflash_inject_kv_input_fusion.argtypes = L.dflash_inject_kv.argtypes
    L.dflash_block_loss.restype = ctypes.c_int
    L.dflash_block_loss.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
    L.dflash_status_str.restype = ctypes.c_char_p
    L.dflash_status_str.argtypes = [ctypes.c_int]
    _LIB = L
    return L


class DFlashError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().dflash_status_str(code).decode()
        super().__init__(f"{where}: {msg} ({code})")
        self.code = code


def check(code: int, where: str) -> None:
    if code != DFLASH_OK:
        raise DFlashError(code, where)
