"""CPU oracle for the DFlash drafting + verification cycle.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
does not, and nothing here imports the GPU library.
"""
from .dflash import (round_bf16, decode_storage, Numerics, rms_norm, silu, rope, rope_angles,  # noqa: F401
                     linear, softmax_rows, block_attention, argmax_lowest, DraftModel, KVCache,
                     fuse, context_kv_rows, inject, draft, verify, cycle)
