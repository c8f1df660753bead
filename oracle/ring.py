"""The per-device ring loop, emulated on the host in fp64 (test only).

"Context parallelism and ring attention", section "Ring attention": each
device keeps its query shard and, step after step, attends to the key/value
block it currently holds, folds the result into a running softmax state and
passes the block on.  Reading for the ring direction (the page only says
"send to the next device"): at step s rank r holds the K/V chunk that started
on rank (r - s) mod R, so step 0 is the rank's own chunk.  The direction
changes only the rounding order.

The sequence is first permuted by a causal load-balancing map (tutorial
section 4 / "Load balance"), cut into R shards, and the per-rank outputs are
concatenated and permuted back.  The result must equal the unsplit attention.
"""

from __future__ import annotations

import numpy as np

from ._arrays import f64, i64
from .attention import attention
from .merge import merge
from .reorder import apply_map, inverse_map, reorder_map


def ring_attention(q, k, v, qid, qpos, kid, kpos, cp_size, kind, stripe=1, scale=None,
                   causal=True, window=(-1, -1), workers=None, return_parts=False):
    q, k, v = f64(q), f64(k), f64(v)
    qid, qpos, kid, kpos = i64(qid), i64(qpos), i64(kid), i64(kpos)
    t = q.shape[1]
    if k.shape[1] != t:
        raise ValueError("the ring emulation assumes self-attention (Tq == Tk)")
    m = reorder_map(t, cp_size, kind, stripe)
    q_r, k_r, v_r = apply_map(q, m), apply_map(k, m), apply_map(v, m)
    qid_r, qpos_r = apply_map(qid, m), apply_map(qpos, m)
    kid_r, kpos_r = apply_map(kid, m), apply_map(kpos, m)
    n = t // cp_size
    o_r = np.zeros_like(q_r)
    lse_r = np.full(q_r.shape[:3], -np.inf)
    parts = {}
    for r in range(cp_size):
        rows = slice(r * n, (r + 1) * n)
        acc = None
        for s in range(cp_size):
            c = (r - s) % cp_size
            cols = slice(c * n, (c + 1) * n)
            part = attention(q_r[:, rows], k_r[:, cols], v_r[:, cols],
                             qid_r[:, rows], qpos_r[:, rows], kid_r[:, cols], kpos_r[:, cols],
                             scale=scale, causal=causal, window=window, workers=workers)
            if return_parts:
                parts[(r, s)] = part
            acc = part if acc is None else merge(acc[0], acc[1], part[0], part[1])
        o_r[:, rows], lse_r[:, rows] = acc
    inv = inverse_map(m)
    out = apply_map(o_r, inv), apply_map(lse_r, inv)
    if return_parts:
        return out, parts
    return out
