"""Causal load-balancing sequence permutations (test infrastructure only).

A map ``m`` of length T gives the reordered sequence as
``reordered[p] = original[m[p]]`` along the sequence axis (axis 1 of every
``[B, T, ...]`` tensor: Q, K, V, segment ids and positions, and the outputs);
the reordered sequence is then cut into ``cp_size`` equal contiguous shards,
shard r belonging to rank r.

* "striped" with stripe size s (TransformerEngine JAX tutorial, section 4,
  ``ReorderStrategy.Striped`` with ``stripe_size``): the sequence is cut into
  stripes of s tokens and stripe j goes to rank j mod R; each rank keeps its
  stripes in their original order.  The pages give no formula; this is the
  plain reading of the strategy's name and parameters.
* "dual_chunk" ("Context parallelism and ring attention", section "Load
  balance": pair early and late pieces on each device): the sequence is cut
  into 2R equal stripes and rank r holds stripe r followed by stripe
  2R-1-r.

Both maps are built here by listing each rank's stripes in turn, not by a
closed-form index formula.
"""

from __future__ import annotations

import numpy as np


def reorder_map(seq_len: int, cp_size: int, kind: str, stripe: int = 1) -> np.ndarray:
    t, r_ = int(seq_len), int(cp_size)
    if kind == "dual_chunk":
        if t % (2 * r_):
            raise ValueError("dual_chunk needs seq_len divisible by 2*cp_size")
        c = t // (2 * r_)
        pieces = []
        for r in range(r_):
            for stripe_index in (r, 2 * r_ - 1 - r):
                pieces.append(np.arange(stripe_index * c, (stripe_index + 1) * c))
        m = np.concatenate(pieces)
    elif kind == "striped":
        s = int(stripe)
        if s <= 0 or t % (r_ * s):
            raise ValueError("striped needs seq_len divisible by cp_size*stripe")
        pieces = []
        for r in range(r_):
            for j in range(r, t // s, r_):
                pieces.append(np.arange(j * s, (j + 1) * s))
        m = np.concatenate(pieces)
    else:
        raise ValueError(f"unknown reorder kind {kind!r}")
    return m.astype(np.int64)


def inverse_map(m) -> np.ndarray:
    """The map that undoes ``m``: ``original[p] = reordered[inv[p]]``."""
    m = np.asarray(m)
    inv = np.empty_like(m)
    inv[m] = np.arange(m.size, dtype=m.dtype)
    return inv


def apply_map(x, m, axis: int = 1):
    """``y`` with ``y[..., p, ...] = x[..., m[p], ...]`` along ``axis``."""
    return np.take(np.asarray(x), np.asarray(m), axis=axis)
