"""Merging partial attention results over disjoint key sets (fp64, test only).

"Context parallelism and ring attention", section "Online softmax": per query
row keep the running maximum score m, the sum z of exponentials taken
relative to m, and the exponential-weighted value sum u; a new block's
(m_b, z_b, u_b) folds in as

    m' = max(m, m_b)
    z' = exp(m - m') z + exp(m_b - m') z_b
    u' = exp(m - m') u + exp(m_b - m') u_b

and the output is u'/z' once all blocks are in.  A fused forward returns
(O, LSE) instead of (m, z, u) ("Implementation: NVIDIA TransformerEngine JAX
Cpp Attention", I/O contract: output and softmax_aux).  Since O = u/z and
exp(LSE) = z exp(m), the pair (m=LSE, z=1, u=O) is a valid state for the same
block, and the fold becomes the log-sum-exp merge below.

Reading for rows with no visible key (the page's update is undefined when
both maxima are -inf): such a row is the identity of the merge, O = 0,
LSE = -inf; merging two of them gives another.
"""

from __future__ import annotations

import numpy as np

from ._arrays import f64


def merge(o_a, lse_a, o_b, lse_b):
    """(O, LSE) of attention over the union of two disjoint key sets.

    ``o_*`` are ``[..., D]``, ``lse_*`` are ``[...]``.  Returns fp64 arrays.
    """
    o_a, o_b = f64(o_a), f64(o_b)
    lse_a, lse_b = f64(lse_a), f64(lse_b)
    lse = np.logaddexp(lse_a, lse_b)
    empty = np.isneginf(lse)
    ref = np.where(empty, 0.0, lse)
    w_a = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - ref))
    w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - ref))
    o = w_a[..., None] * o_a + w_b[..., None] * o_b
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


def state_from_output(o, lse):
    """(m, z, u) state equivalent to a block's (O, LSE)."""
    o, lse = f64(o), f64(lse)
    live = np.isfinite(lse)
    m = np.where(live, lse, -np.inf)
    z = live.astype(np.float64)
    u = np.where(live[..., None], o, 0.0)
    return m, z, u


def state_to_output(m, z, u):
    """(O, LSE) of a finished (m, z, u) state: O = u/z, LSE = m + ln z."""
    live = z > 0
    zs = np.where(live, z, 1.0)
    o = np.where(live[..., None], u / zs[..., None], 0.0)
    lse = np.where(live, m + np.log(zs), -np.inf)
    return o, lse


def fold_mzu(state, block):
    """One online-softmax update of (m, z, u) by a block's (m_b, z_b, u_b)."""
    m, z, u = state
    m_b, z_b, u_b = block
    m_new = np.maximum(m, m_b)
    ref = np.where(np.isneginf(m_new), 0.0, m_new)
    a = np.where(np.isneginf(m), 0.0, np.exp(m - ref))
    a_b = np.where(np.isneginf(m_b), 0.0, np.exp(m_b - ref))
    return m_new, a * z + a_b * z_b, a[..., None] * u + a_b[..., None] * u_b
