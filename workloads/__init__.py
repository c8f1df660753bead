"""Seeded synthetic inputs for the blockwise online-softmax attention forward.

This module only *draws* inputs: Q/K/V values and packed-sequence metadata
(segment ids and positions).  It holds none of the attention arithmetic, no
mask predicate, no reorder map and no merge rule, so both the HIP path and the
fp64 oracle can be fed from it without sharing any of the method.

Workload shapes follow the TransformerEngine JAX tutorial "Context-Parallel
Attention with TransformerEngine", section 1 (packed THD inputs): B=2 rows of
65536 tokens, four 16384-token segment slots per row with 12288 valid tokens
(ids 1..4) followed by 4096 padding tokens (id 0), positions counting 0..16383
inside every slot, 128 query heads over 8 K/V heads, head_dim 128, bf16 values
drawn from N(0, 1).  The smaller workloads keep that recipe at other sizes.
"""

from .configs import CONFIGS, Workload, get
from .generate import (
    packed_metadata,
    qkv,
    random_layout,
    random_qkv,
)

__all__ = [
    "CONFIGS",
    "Workload",
    "get",
    "packed_metadata",
    "qkv",
    "random_layout",
    "random_qkv",
]
