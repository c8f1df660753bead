"""fp64 CPU oracle for blockwise online-softmax attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table
or helper with the HIP library; the two meet only in the seeded input
generators of ``workloads/``, which hold no attention arithmetic.

What it computes, and where that is defined:

* ``attention``/``attention_rows``: exact masked softmax attention
  O = softmax(scale * Q K^T + M) V with the natural-log log-sum-exp of the
  masked, scaled scores as the softmax aux.  Formula: "Context parallelism and
  ring attention", section "The attention problem"; scale head_dim**-0.5 and
  the padding+causal mask, sliding window and vanilla softmax from the
  TransformerEngine JAX tutorial "Context-Parallel Attention", section 3
  (fused attention call); segment ids / positions from its section 1; the
  (output, softmax_aux) pair from "Implementation: NVIDIA TransformerEngine JAX
  Cpp Attention", I/O contract, outputs.  V may carry its own head dim (the
  tutorial's "Next steps" section points to single-GPU attention with
  DeepSeek-style MLA head dimensions); O then has V's head dim and the default
  scale stays Q/K's head_dim**-0.5.
* ``merge``/``fold_mzu``: combining partial results over disjoint key blocks,
  "Context parallelism and ring attention", section "Online softmax".
* ``reorder_map``: causal load-balancing permutations (tutorial section 4,
  striped; dual-chunk pairing of stripe i with stripe 2R-1-i as described in
  "Context parallelism and ring attention", section "Load balance").
* ``classify_tiles_exact``/``visible_pairs``: skip / full / partial blocks,
  "Context parallelism and ring attention", section "Causal attention".
* ``ring_attention``: the per-device ring loop, section "Ring attention".
* ``attention_backward`` (and per-row / per-key samples): dQ, dK, dV of the
  attention above by the chain rule of its definition; the pages time the
  forward together with its backward (tutorial section 5) but print no
  backward formula.

Every function is pinned by the ``-m "not gpu"`` tests against closed forms,
invariants, a library routine (torch's scaled-dot-product attention on the
CPU in fp64) and scalar brute force; nothing is "parity unpinned".
"""

from .attention import attention, attention_rows, visible
from .backward import attention_backward, backward_key_rows, backward_query_rows
from .merge import fold_mzu, merge, state_from_output, state_to_output
from .reorder import apply_map, inverse_map, reorder_map
from .ring import ring_attention
from .tiles import classify_tiles_exact, tile_class_counts, visible_pairs

__all__ = [
    "attention", "attention_rows", "visible",
    "attention_backward", "backward_query_rows", "backward_key_rows",
    "merge", "fold_mzu", "state_from_output", "state_to_output",
    "reorder_map", "inverse_map", "apply_map",
    "ring_attention",
    "classify_tiles_exact", "tile_class_counts", "visible_pairs",
]
