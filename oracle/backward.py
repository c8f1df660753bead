"""Gradients of exact masked GQA softmax attention in fp64 (test infrastructure only).

The forward is O = softmax(scale * Q K^T + M) V per head ("Context parallelism
and ring attention", section "The attention problem"; mask, scale and GQA
pairing as in ``attention``).  The TransformerEngine JAX tutorial times it
together with its backward (section 5, forward+backward), and the
implementation page lists the backward primitives next to the forward ones.
No page prints the backward formulas; they are the chain rule of that
definition, written out per query head h reading K/V head g:

    S  = scale * Q_h K_g^T + M,   P = softmax(S) row by row (a row with no
                                      visible key is all zeros)
    dV_g += P^T dO_h
    dP  = dO_h V_g^T
    dS  = P * (dP - rowsum(P * dP))         (rowsum(P * dP) = rowsum(dO_h * O_h))
    dQ_h = scale * dS K_g
    dK_g += scale * dS^T Q_h

dK and dV of a K/V head sum over the query heads of its group.  Every row is
one plain softmax over its whole visible key set; no blockwise evaluation.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from ._arrays import f64, i64
from .attention import _default_workers, _take_keys, visible


def _row_softmax(s, vis):
    """Masked row softmax; rows without a visible entry become zeros."""
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    live = np.isfinite(m)
    e = np.exp(s - np.where(live, m, 0.0))
    z = e.sum(axis=-1, keepdims=True)
    return np.where(live, e / np.where(live, z, 1.0), 0.0)


def attention_backward(q, k, v, do, qid, qpos, kid, kpos, scale=None, causal=True,
                       window=(-1, -1), q_block=256, workers=None):
    """(dQ, dK, dV) in fp64 for q ``[B,Tq,Hq,D]``, k/v ``[B,Tk,Hkv,D]``, dO like q.

    Work is spread over host threads by (batch row, K/V head); each job owns
    its dK/dV slice, so no two threads write the same element.
    """
    q, k, v, do = f64(q), f64(k), f64(v), f64(do)
    qid, qpos, kid, kpos = i64(qid), i64(qpos), i64(kid), i64(kpos)
    b_, tq, hq, d = q.shape
    hkv = k.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    grp = hq // hkv
    if scale is None:
        scale = d ** -0.5
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)

    def one(job):
        b, g = job
        for i0 in range(0, tq, q_block):
            i1 = min(i0 + q_block, tq)
            vis = visible(qid[b, i0:i1], qpos[b, i0:i1], kid[b], kpos[b], causal, window)
            cand = np.nonzero(vis.any(axis=0))[0]
            if cand.size == 0:
                continue
            vis = vis[:, cand]
            kc, vc = k[b, cand, g, :], v[b, cand, g, :]
            for h in range(g * grp, (g + 1) * grp):
                qh, doh = q[b, i0:i1, h, :], do[b, i0:i1, h, :]
                p = _row_softmax(scale * (qh @ kc.T), vis)
                dv[b, cand, g, :] += p.T @ doh
                dp = doh @ vc.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, i0:i1, h, :] = scale * (ds @ kc)
                dk[b, cand, g, :] += scale * (ds.T @ qh)

    jobs = [(b, g) for b in range(b_) for g in range(hkv)]
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
    return dq, dk, dv


def _rows_dq(qrows, dorows, k, v, qid, qpos, kid, kpos, rows, scale, causal=True,
             window=(-1, -1)):
    """dQ ``[n, Hq, D]`` of single query rows: ``qrows[n]`` and ``dorows[n]``
    (``[Hq, D]``, ``[Hq, Dv]``) are the query and output gradient at
    ``rows[n] = (b, t)``; metadata int64 ``[B, T]``; k, v indexable."""
    n_rows, hq, d = qrows.shape
    hkv = k.shape[2]
    grp = hq // hkv
    out = np.zeros((n_rows, hq, d))
    for n, (b, t) in enumerate(rows):
        vis = visible(qid[b, t:t + 1], qpos[b, t:t + 1], kid[b], kpos[b], causal, window)[0]
        cand = np.nonzero(vis)[0]
        if cand.size == 0:
            continue
        for g in range(hkv):
            kc, vc = _take_keys(k, b, cand, g), _take_keys(v, b, cand, g)
            for h in range(g * grp, (g + 1) * grp):
                qh, doh = f64(qrows[n, h]), f64(dorows[n, h])
                p = _row_softmax(scale * (kc @ qh)[None, :], np.ones((1, cand.size), bool))[0]
                dp = vc @ doh
                ds = p * (dp - (p * dp).sum())
                out[n, h] = scale * (ds @ kc)
    return out


def backward_query_rows(q, k, v, do, qid, qpos, kid, kpos, rows, scale=None, causal=True,
                        window=(-1, -1), workers=None):
    """dQ of selected query rows ``[(b, t), ...]``: ``[len(rows), Hq, D]``.

    dQ of a row depends only on that row and the keys it sees, so full-size
    problems can be checked on a sample; a large sample is spread over worker
    processes running this same row function (``workers``, as in
    ``attention_rows``).
    """
    from .attention import _gather_rows
    rows = [(int(b), int(t)) for b, t in rows]
    d = q.shape[3]
    if scale is None:
        scale = d ** -0.5
    if not rows:
        return np.zeros((0, q.shape[2], d))
    qrows, dorows = _gather_rows(q, rows), _gather_rows(do, rows)
    if workers is None:
        from .pool import pool_workers
        workers = pool_workers() if len(rows) >= 32 else 1
    if workers > 1 and len(rows) > 1:
        from .pool import RowPool
        with RowPool(k, v, qid, qpos, kid, kpos, workers) as pool:
            return pool.dq(qrows, dorows, rows, scale=scale, causal=causal, window=window)
    return _rows_dq(qrows, dorows, k, v, i64(qid), i64(qpos), i64(kid), i64(kpos), rows,
                    scale, causal, window)


def backward_key_rows(q, k, v, do, qid, qpos, kid, kpos, keys, scale=None, causal=True,
                      window=(-1, -1)):
    """(dK, dV) of selected key rows ``[(b, t), ...]``: ``[len(keys), Hkv, D]`` and
    ``[len(keys), Hkv, Dv]`` (dV has V's head dim).

    A key's gradients gather every query that sees it; each such query's
    softmax needs that query's whole visible key set.
    """
    b_, tq, hq, d = q.shape
    hkv = k.shape[2]
    grp = hq // hkv
    if scale is None:
        scale = d ** -0.5
    dk = np.zeros((len(keys), hkv, d))
    dv = np.zeros((len(keys), hkv, v.shape[3]))
    for n, (b, j) in enumerate(keys):
        seen = visible(i64(qid[b]), i64(qpos[b]), i64(kid[b, j:j + 1]), i64(kpos[b, j:j + 1]),
                       causal, window)[:, 0]
        rows = np.nonzero(seen)[0]
        if rows.size == 0:
            continue
        vis = visible(i64(qid[b, rows]), i64(qpos[b, rows]), i64(kid[b]), i64(kpos[b]), causal,
                      window)
        cand = np.nonzero(vis.any(axis=0))[0]
        vis = vis[:, cand]
        col = int(np.nonzero(cand == j)[0][0])
        for g in range(hkv):
            kc, vc = f64(k[b, cand, g, :]), f64(v[b, cand, g, :])
            for h in range(g * grp, (g + 1) * grp):
                qh, doh = f64(q[b, rows, h, :]), f64(do[b, rows, h, :])
                p = _row_softmax(scale * (qh @ kc.T), vis)
                dp = doh @ vc.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dv[n, g] += p[:, col] @ doh
                dk[n, g] += scale * (ds[:, col] @ qh)
    return dk, dv
