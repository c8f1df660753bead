"""Exact masked GQA softmax attention in fp64 (test infrastructure only).

Definition ("Context parallelism and ring attention", section "The attention
problem"): for one head, O = softmax(Q K^T * scale + M) V, where M is 0 on a
visible (query, key) pair and -inf elsewhere.  The scale is head_dim**-0.5
(TransformerEngine JAX tutorial, section 3, ``scaling_factor``).  Readings
taken where the pages leave a point open:

* A pair is visible when both tokens carry the same nonzero segment id in the
  same batch row (id 0 marks padding, tutorial section 1), the key position is
  not after the query position when causal (``PADDING_CAUSAL_MASK``), and the
  key lies inside the sliding window ``(left, right)`` (tutorial section 3,
  ``window_size``) read inclusively on positions:
  ``qpos - left <= kpos <= qpos + right``, with -1 meaning unbounded.
  Positions are the per-token ``segment_pos`` values, never array indices,
  so the rule survives any reordering of the sequence.
* Query head h reads K/V head ``h // (Hq // Hkv)`` (contiguous GQA groups).
* A query with no visible key gets O = 0 and LSE = -inf.
* The softmax aux is the natural-log log-sum-exp of the masked, scaled
  scores, LSE = m + ln(sum_j exp(s_j - m)).

Rows are independent, so rows may be evaluated in any grouping; keys outside
a row's visible set contribute exactly zero, so only keys visible to some row
of a group are gathered.  No online or blockwise softmax is used here: every
row is one plain softmax over its whole visible key set.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from ._arrays import f64, i64


def visible(qid, qpos, kid, kpos, causal=True, window=(-1, -1)):
    """Boolean ``[nq, nk]`` visibility of every (query, key) pair of one batch row."""
    qid = i64(qid)[:, None]
    qpos = i64(qpos)[:, None]
    kid = i64(kid)[None, :]
    kpos = i64(kpos)[None, :]
    vis = (qid != 0) & (kid != 0) & (qid == kid)
    if causal:
        vis &= kpos <= qpos
    left, right = int(window[0]), int(window[1])
    if left >= 0:
        vis &= (qpos - kpos) <= left
    if right >= 0:
        vis &= (kpos - qpos) <= right
    return vis


def _softmax_rows(qh, kc, vc, vis, scale):
    """One plain softmax per row.

    qh ``[n, G, D]`` (n query tokens of one head group), kc ``[m, D]`` and vc
    ``[m, Dv]`` (the group's K/V head at m candidate keys), vis ``[n, m]``.
    Returns O ``[n, G, Dv]`` and LSE ``[n, G]``.
    """
    n, g, d = qh.shape
    dv = vc.shape[1]
    o = np.zeros((n, g, dv))
    lse = np.full((n, g), -np.inf)
    if kc.shape[0] == 0:
        return o, lse
    s = (qh.reshape(n * g, d) @ kc.T).reshape(n, g, -1) * scale
    s = np.where(vis[:, None, :], s, -np.inf)
    m = s.max(axis=2)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[:, :, None])           # masked entries give exp(-inf) = 0
    z = e.sum(axis=2)
    u = (e.reshape(n * g, -1) @ vc).reshape(n, g, dv)
    o = np.where(live[:, :, None], u / np.where(live, z, 1.0)[:, :, None], 0.0)
    lse = np.where(live, m_safe + np.log(np.where(live, z, 1.0)), -np.inf)
    return o, lse


def _default_workers():
    return max(1, len(os.sched_getaffinity(0)))


def attention(q, k, v, qid, qpos, kid, kpos, scale=None, causal=True, window=(-1, -1),
              q_block=128, workers=None):
    """Exact attention over whole tensors.

    q ``[B, Tq, Hq, D]``, k ``[B, Tk, Hkv, D]``, v ``[B, Tk, Hkv, Dv]``, metadata
    ``[B, T]``.  Returns fp64 ``O [B, Tq, Hq, Dv]`` and ``LSE [B, Tq, Hq]``.  V's
    head dim may differ from Q's and K's (the tutorial's "Next steps" section
    names DeepSeek-style MLA head dimensions); the default scale is D**-0.5 of Q/K.
    Work is spread over host threads by (batch row, query block); numpy
    releases the GIL inside its kernels.
    """
    q, k, v = f64(q), f64(k), f64(v)
    qid, qpos, kid, kpos = i64(qid), i64(qpos), i64(kid), i64(kpos)
    b_, tq, hq, d = q.shape
    hkv = k.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    grp = hq // hkv
    if scale is None:
        scale = d ** -0.5
    o = np.zeros((b_, tq, hq, v.shape[3]))
    lse = np.full((b_, tq, hq), -np.inf)

    def one(job):
        b, i0 = job
        i1 = min(i0 + q_block, tq)
        vis = visible(qid[b, i0:i1], qpos[b, i0:i1], kid[b], kpos[b], causal, window)
        cand = np.nonzero(vis.any(axis=0))[0]
        if cand.size == 0:
            return
        vis = vis[:, cand]
        for g in range(hkv):
            qh = q[b, i0:i1, g * grp:(g + 1) * grp, :]
            og, lg = _softmax_rows(qh, k[b, cand, g, :], v[b, cand, g, :], vis, scale)
            o[b, i0:i1, g * grp:(g + 1) * grp, :] = og
            lse[b, i0:i1, g * grp:(g + 1) * grp] = lg

    jobs = [(b, i0) for b in range(b_) for i0 in range(0, tq, q_block)]
    nw = workers or _default_workers()
    if nw <= 1 or len(jobs) <= 1:
        for j in jobs:
            one(j)
    else:
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(1)
        except ImportError:  # pragma: no cover
            limiter = None
        try:
            with ThreadPoolExecutor(nw) as ex:
                list(ex.map(one, jobs))
        finally:
            if limiter is not None:
                limiter.restore_original_limits()
    return o, lse


def _take_keys(x, b, cand, g):
    """fp64 ``[len(cand), D]`` rows of K/V head g in batch row b."""
    if hasattr(x, "detach"):
        import torch
        idx = torch.from_numpy(np.ascontiguousarray(cand)).to(x.device)
        return f64(x[b].index_select(0, idx)[:, g, :])
    return f64(np.asarray(x)[b, cand, g, :])


def _gather_rows(x, rows):
    """fp64 ``[len(rows), H, D]``: the (batch, token) rows of a [B, T, H, D] array-like."""
    if hasattr(x, "detach"):
        import torch
        bi = torch.tensor([r[0] for r in rows], dtype=torch.int64, device=x.device)
        ti = torch.tensor([r[1] for r in rows], dtype=torch.int64, device=x.device)
        return f64(x[bi, ti])
    a = np.asarray(x)
    return f64(a[[r[0] for r in rows], [r[1] for r in rows]])


def _rows_forward(qrows, k, v, qid, qpos, kid, kpos, rows, scale, causal=True, window=(-1, -1)):
    """Exact attention of single query rows, one plain softmax per row and head.

    ``qrows[n]`` ``[Hq, D]`` is the query at ``rows[n] = (b, i)``; the metadata
    are int64 arrays ``[B, T]``; k, v are indexable ``[B, Tk, Hkv, D(v)]``.
    """
    n_rows, hq = qrows.shape[0], qrows.shape[1]
    hkv = k.shape[2]
    grp = hq // hkv
    o = np.zeros((n_rows, hq, v.shape[3]))
    lse = np.full((n_rows, hq), -np.inf)
    for n, (b, i) in enumerate(rows):
        vis = visible(qid[b, i:i + 1], qpos[b, i:i + 1], kid[b], kpos[b], causal, window)
        cand = np.nonzero(vis[0])[0]
        if cand.size == 0:
            continue
        qrow = f64(qrows[n])                      # [Hq, D]
        for g in range(hkv):
            kc = _take_keys(k, b, cand, g)
            vc = _take_keys(v, b, cand, g)
            og, lg = _softmax_rows(qrow[None, g * grp:(g + 1) * grp, :], kc, vc,
                                   np.ones((1, cand.size), bool), scale)
            o[n, g * grp:(g + 1) * grp] = og[0]
            lse[n, g * grp:(g + 1) * grp] = lg[0]
    return o, lse


def attention_rows(q, k, v, qid, qpos, kid, kpos, rows, scale=None, causal=True,
                   window=(-1, -1), workers=None):
    """Exact attention for selected query rows only.

    ``rows`` is a sequence of (batch, token) pairs.  Returns fp64 O
    ``[n, Hq, Dv]`` and LSE ``[n, Hq]`` for those rows, every head.  Used where
    the full output is too large for the oracle; K and V may be any array-like
    (they are only indexed, then widened).  Rows are independent, so a large
    sample is spread over worker processes (``workers``; default: the host
    cores for 32 rows or more, else this process) that run the same row
    function on shared copies of K, V and the metadata.
    """
    rows = [(int(b), int(i)) for b, i in rows]
    d = q.shape[3]
    if scale is None:
        scale = d ** -0.5
    qrows = _gather_rows(q, rows) if rows else np.zeros((0, q.shape[2], d))
    if workers is None:
        from .pool import pool_workers
        workers = pool_workers() if len(rows) >= 32 else 1
    if workers > 1 and len(rows) > 1:
        from .pool import RowPool
        with RowPool(k, v, qid, qpos, kid, kpos, workers) as pool:
            return pool.forward(qrows, rows, scale=scale, causal=causal, window=window)
    return _rows_forward(qrows, k, v, i64(qid), i64(qpos), i64(kid), i64(kpos), rows, scale,
                         causal, window)
