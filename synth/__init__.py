"""Seeded synthetic inputs shared by the oracle and the HIP path.

This package holds shapes and random-number recipes only: it performs none of
the drafter's arithmetic (no norms, projections, attention, argmax or
verification).  Both the CPU oracle (``oracle/``) and the GPU binding
(``block_diffusion_drafter_states_amd``) draw their inputs from here, so the two
sides see bit-identical weights, features, caches and token ids.
"""
from .configs import Config, CONFIGS, get_config, tiny_config  # noqa: F401
from . import gen  # noqa: F401
