"""Seeded synthetic inputs for MLA absorbed decode.

This package only draws random numbers, rounds them to the storage formats
(bf16, fp32, OCP FP8 E4M3 with a per-token scale) and lays the cached rows
out in memory (contiguous or paged in 64-token blocks).  It contains none of
the attention arithmetic: no RoPE, no projection, no softmax.  Both the CPU
oracle and the GPU path consume what it produces.
"""

from .configs import (BLOCK_TOKENS, CONFIGS, HEADLINE, OUT_FUSED_CONFIGS, PREFILL_CONFIGS, MLAConfig,
                      scaled)
from .generate import AppendInputs, MLAInputs, OutProjInputs, Pool

__all__ = [
    "AppendInputs",
    "BLOCK_TOKENS",
    "CONFIGS",
    "HEADLINE",
    "MLAConfig",
    "MLAInputs",
    "OUT_FUSED_CONFIGS",
    "OutProjInputs",
    "PREFILL_CONFIGS",
    "Pool",
    "scaled",
]
