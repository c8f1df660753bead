"""Block classification and visible-pair counts by brute force (test only).

"Context parallelism and ring attention", section "Causal attention": a block
of (query, key) pairs is skipped when nothing in it is visible, processed
without a mask when everything in it is visible, and masked otherwise.  Here
the class of a tile of ``bm`` query tokens by ``bn`` key tokens is decided
exactly from the full visibility mask over the tile's in-range pairs
(0 = skip: none visible, 2 = full: all visible, 1 = partial).  Tiles past the
end of the sequence are cut short, never padded with invisible pairs.  The
mask does not depend on the head, so the map is indexed by
(batch row, query tile, key tile).
"""

from __future__ import annotations

import numpy as np

from ._arrays import i64
from .attention import visible

SKIP, PARTIAL, FULL = 0, 1, 2


def classify_tiles_exact(qid, qpos, kid, kpos, bm, bn, causal=True, window=(-1, -1)):
    """int8 ``[B, ceil(Tq/bm), ceil(Tk/bn)]`` tile classes."""
    qid, qpos, kid, kpos = i64(qid), i64(qpos), i64(kid), i64(kpos)
    b_, tq = qid.shape
    tk = kid.shape[1]
    nqt = -(-tq // bm)
    nkt = -(-tk // bn)
    out = np.zeros((b_, nqt, nkt), np.int8)
    pad = nkt * bn - tk
    for b in range(b_):
        for qt in range(nqt):
            i0, i1 = qt * bm, min((qt + 1) * bm, tq)
            vis = visible(qid[b, i0:i1], qpos[b, i0:i1], kid[b], kpos[b], causal, window)
            # out-of-range key slots count as invisible for "any" and visible for "all"
            any_v = np.pad(vis, ((0, 0), (0, pad)), constant_values=False)
            all_v = np.pad(vis, ((0, 0), (0, pad)), constant_values=True)
            some = any_v.reshape(i1 - i0, nkt, bn).any(axis=(0, 2))
            every = all_v.reshape(i1 - i0, nkt, bn).all(axis=(0, 2))
            out[b, qt] = np.where(every, FULL, np.where(some, PARTIAL, SKIP))
    return out


def tile_class_counts(classes):
    """(skip, partial, full) totals of a class map."""
    c = np.asarray(classes)
    return int((c == SKIP).sum()), int((c == PARTIAL).sum()), int((c == FULL).sum())


def visible_pairs(qid, qpos, kid, kpos, causal=True, window=(-1, -1), q_block=1024):
    """Number of visible (query, key) pairs in each batch row (int64 ``[B]``)."""
    qid, qpos, kid, kpos = i64(qid), i64(qpos), i64(kid), i64(kpos)
    b_, tq = qid.shape
    out = np.zeros(b_, np.int64)
    for b in range(b_):
        for i0 in range(0, tq, q_block):
            i1 = min(i0 + q_block, tq)
            out[b] += int(visible(qid[b, i0:i1], qpos[b, i0:i1], kid[b], kpos[b],
                                  causal, window).sum())
    return out
