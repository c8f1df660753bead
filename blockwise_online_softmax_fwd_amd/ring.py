"""One-GPU ring driver: context-parallel ring attention's per-device loop, run
for every rank in turn on one GPU.

"Context parallelism and ring attention", section "Ring attention": a device
keeps its query shard and, at each step, attends to the key/value block it
holds, folds the result into a running softmax state ("Online softmax") and
passes the block on; after R steps every local query has seen every allowed
key.  Here the exchange is replaced by indexing: at step s rank r holds the
chunk that started on rank (r - s) mod R (step 0 is its own chunk).  Before the
loop the sequence is permuted for causal load balance and cut into R shards
(TransformerEngine JAX tutorial, section 4); afterwards the output and the LSE
are permuted back.  Every step is a call into libringattn; this module only
slices views and orders the calls.

The all-gather strategy (TransformerEngine JAX tutorial, sections 4 and 5;
"Context parallelism and ring attention", "Communication choices") is the
other per-device computation: each rank keeps its query shard of the
striped reorder and attends, in a single call, to the whole gathered K/V (in
reordered order; the mask works on segment ids and positions, so the order
of the keys does not matter).  No partials, no merge.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import ringattn as ra


@dataclass
class RingBuffers:
    """Device buffers of one ring forward, reusable across calls of one shape."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    ids: torch.Tensor
    pos: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    acc: torch.Tensor
    acc_lse: torch.Tensor
    part: torch.Tensor
    part_lse: torch.Tensor
    workspace: torch.Tensor | None = None
    # split workspaces (ra_attn_fwd_ex): one packed-K/V buffer per K/V chunk and
    # a schedule buffer for calls without a plan
    kv_ws: dict = field(default_factory=dict)
    sched_ws: torch.Tensor | None = None

    @classmethod
    def like(cls, q, k, ids, cp_size, partial_dtype=torch.float32, out_dtype=None, partials=True,
             v=None):
        """Buffers for inputs shaped like q, k (and v, whose head dim O takes;
        k's when v is not given)."""
        b, t, hq, _ = q.shape
        d = (k if v is None else v).shape[3]
        n = t // cp_size if partials else 0
        dev = q.device
        od = q.dtype if out_dtype is None else out_dtype
        return cls(
            q=torch.empty_like(q), k=torch.empty_like(k),
            v=torch.empty_like(k if v is None else v),
            ids=torch.empty_like(ids), pos=torch.empty_like(ids),
            o=torch.empty((b, t, hq, d), dtype=od, device=dev),
            lse=torch.empty((b, t, hq), dtype=torch.float32, device=dev),
            acc=torch.empty((b, n, hq, d), dtype=partial_dtype, device=dev),
            acc_lse=torch.empty((b, n, hq), dtype=torch.float32, device=dev),
            part=torch.empty((b, n, hq, d), dtype=partial_dtype, device=dev),
            part_lse=torch.empty((b, n, hq), dtype=torch.float32, device=dev),
        )


def reorder_inputs(q, k, v, ids, pos, cp_size, kind, stripe_size, bufs: RingBuffers, with_q=True):
    if with_q:
        ra.reorder(q, cp_size, kind, stripe_size, out=bufs.q)
    ra.reorder(k, cp_size, kind, stripe_size, out=bufs.k)
    ra.reorder(v, cp_size, kind, stripe_size, out=bufs.v)
    ra.reorder(ids, cp_size, kind, stripe_size, out=bufs.ids)
    ra.reorder(pos, cp_size, kind, stripe_size, out=bufs.pos)


class _Prepared:
    """The split workspaces of one driver call (``ra_attn_fwd_ex``).

    Every K/V chunk is packed by the first call that reads it and reused by the
    others (K/V do not change during the driver call; a new driver call packs
    again).  Schedules -- tile lists, a function of the layout, the mask and
    the tile shape only -- live in the plan when there is one, keyed by
    (rank, step, stripes) and the tile-shape inputs, and are computed once per
    plan; without a plan every call writes one shared schedule buffer anew.
    """

    def __init__(self, bufs, plan, desc_full, key_extra):
        self.bufs, self.plan = bufs, plan
        self.sched_bytes, self.kv_bytes = ra.workspace_parts(desc_full)
        self.key_extra = key_extra
        self.packed = set()
        dev = bufs.q.device
        for c in list(bufs.kv_ws):
            if bufs.kv_ws[c].numel() < self.kv_bytes:
                del bufs.kv_ws[c]
        if plan is None and (bufs.sched_ws is None or bufs.sched_ws.numel() < self.sched_bytes):
            bufs.sched_ws = torch.empty(max(1, self.sched_bytes), dtype=torch.uint8, device=dev)
        self.dev = dev

    def get(self, key, chunk):
        """``(schedule_ws, kv_ws, flags)`` for a call on ``chunk``, and a callback
        that records the call's buffers as written once it has been enqueued."""
        flags = 0
        kv = self.bufs.kv_ws.get(chunk)
        if kv is None:
            kv = torch.empty(max(1, self.kv_bytes), dtype=torch.uint8, device=self.dev)
            self.bufs.kv_ws[chunk] = kv
        if chunk in self.packed:
            flags |= ra.FWD_KV_READY
        if self.plan is None:
            sched = self.bufs.sched_ws
            skey = None
        else:
            skey = (key, self.key_extra, str(self.dev))
            sched = self.plan.schedules.get(skey)
            if sched is None:
                sched = torch.empty(max(1, self.sched_bytes), dtype=torch.uint8, device=self.dev)
                self.plan.schedules[skey] = sched
            if skey in self.plan.ready:
                flags |= ra.FWD_SCHEDULE_READY

        def done():
            self.packed.add(chunk)
            if skey is not None:
                self.plan.ready.add(skey)
        return (sched, kv, flags), done


def rank_steps(rank, cp_size, bufs: RingBuffers, *, scale=None, causal=True, window=(-1, -1),
               step_hook=None, fused=True, steps=None, final=None, prep=None):
    """Rank ``rank``'s R ring steps on the reordered buffers; the merged result
    lands in rank's shard of ``bufs.o`` / ``bufs.lse`` (reordered order).

    ``fused``: each step after the first folds its block into the running
    partial inside the forward's epilogue (``attn_fwd_accumulate``, in place in
    the fp32 partial, the last step writing the final output); otherwise every
    step writes its own partial and ``attn_merge`` folds it in.  ``final``
    (fused only): ``(o_lo, lse_lo, split)`` -- the last step writes its output
    there instead of ``bufs.o``, ``split`` as in ``attn_fwd`` (how the
    dual-chunk inverse reorder is folded into the last step)."""
    if fused:
        return _rank_steps_fused(rank, cp_size, bufs, scale, causal, window, step_hook, steps,
                                 final, prep)
    t = bufs.q.shape[1]
    n = t // cp_size
    rows = slice(rank * n, (rank + 1) * n)
    q_r, id_r, pos_r = bufs.q[:, rows], bufs.ids[:, rows], bufs.pos[:, rows]
    o_r, lse_r = bufs.o[:, rows], bufs.lse[:, rows]
    for s in range(cp_size):
        c = (rank - s) % cp_size
        cols = slice(c * n, (c + 1) * n)
        if cp_size == 1:
            dst, dst_lse = o_r, lse_r
        elif s == 0:
            dst, dst_lse = bufs.acc, bufs.acc_lse
        else:
            dst, dst_lse = bufs.part, bufs.part_lse
        prepared, done = prep.get((rank, s, (0, 1)), c) if prep else (None, None)
        if step_hook:
            step_hook("attn_fwd", rank, s, True)
        _, _ = ra.attn_fwd(q_r, bufs.k[:, cols], bufs.v[:, cols], id_r, pos_r, bufs.ids[:, cols],
                           bufs.pos[:, cols], scale=scale, causal=causal, window=window,
                           out_dtype=dst.dtype, out=dst, lse=dst_lse, workspace=bufs.workspace,
                           prepared=prepared)
        if done:
            done()
        if step_hook:
            step_hook("attn_fwd", rank, s, False)
        if s == 0:
            continue
        last = s == cp_size - 1
        if step_hook:
            step_hook("attn_merge", rank, s, True)
        ra.attn_merge(bufs.acc, bufs.acc_lse, bufs.part, bufs.part_lse,
                      out=o_r if last else bufs.acc, lse_out=lse_r if last else bufs.acc_lse)
        if step_hook:
            step_hook("attn_merge", rank, s, False)


def _rank_steps_fused(rank, cp_size, bufs, scale, causal, window, step_hook, steps=None,
                      final=None, prep=None):
    t = bufs.q.shape[1]
    n = t // cp_size
    rows = slice(rank * n, (rank + 1) * n)
    q_r, id_r, pos_r = bufs.q[:, rows], bufs.ids[:, rows], bufs.pos[:, rows]
    if final is None:
        final = (bufs.o[:, rows], bufs.lse[:, rows], None)
    steps = list(range(cp_size)) if steps is None else steps
    for i, s in enumerate(steps):
        c = (rank - s) % cp_size
        cols = slice(c * n, (c + 1) * n)
        args = (q_r, bufs.k[:, cols], bufs.v[:, cols], id_r, pos_r, bufs.ids[:, cols],
                bufs.pos[:, cols])
        last = i == len(steps) - 1
        dst, dst_lse, split = final if last else (bufs.acc, bufs.acc_lse, None)
        prepared, done = prep.get((rank, s, (0, 1)), c) if prep else (None, None)
        if step_hook:
            step_hook("attn_fwd", rank, s, True)
        if i == 0:
            ra.attn_fwd(*args, scale=scale, causal=causal, window=window, out_dtype=dst.dtype,
                        out=dst, lse=dst_lse, workspace=bufs.workspace, split=split,
                        prepared=prepared)
        else:
            ra.attn_fwd_accumulate(*args, bufs.acc, bufs.acc_lse, scale=scale, causal=causal,
                                   window=window, out=dst, lse=dst_lse, workspace=bufs.workspace,
                                   split=split, prepared=prepared)
        if done:
            done()
        if step_hook:
            step_hook("attn_fwd", rank, s, False)


def _layout_fingerprint(ids, pos):
    """Two 64-bit position-weighted sums of the segment ids and positions
    (computed where the tensors live; wrapping int64 arithmetic), to tell one
    segment layout from another."""
    t = ids.shape[1]
    w = torch.arange(1, t + 1, device=ids.device, dtype=torch.int64)
    a = ids.to(torch.int64) * 1000003 + pos.to(torch.int64) * 7919 + 1
    h1 = (a * (w * 2654435761 + 97)).sum(dim=1)
    h2 = ((a ^ (a >> 7)) * (w * w + 31337)).sum(dim=1)
    return tuple(int(x) for x in torch.stack([h1, h2], 1).flatten().tolist())


class RingPlan:
    """The ring schedule of one segment layout and mask (see :func:`ring_plan`).

    ``counts``: host ``int64 [R, R]`` (rank, step), or ``[R, 2, R]`` (rank,
    dual-chunk stripe, step) -- the visible pairs of every block.  The plan
    records what it was computed from (shape, shard count, reorder, mask and a
    fingerprint of the ids and positions); :func:`ring_forward` refuses a plan
    made for anything else, since it would skip blocks that hold visible
    pairs.  Tensors already checked (same storage, unmodified since) are not
    fingerprinted again, so the steady state adds no device synchronisation.
    """

    def __init__(self, counts, ids, pos, cp_size, kind, stripe_size, causal, window):
        self.counts = counts
        self.meta = (tuple(ids.shape), int(cp_size), ra._kind_code(kind),
                     int(stripe_size) if ra._kind_code(kind) == ra.STRIPED else 1,
                     bool(causal), (int(window[0]), int(window[1])))
        self.fingerprint = _layout_fingerprint(ids, pos)
        self._seen = {self._token(ids, pos)}
        # device schedules of the ring's calls on this layout (see _Prepared)
        self.schedules = {}
        self.ready = set()

    @staticmethod
    def _token(ids, pos):
        return (ids.data_ptr(), ids._version, tuple(ids.stride()), pos.data_ptr(), pos._version,
                tuple(pos.stride()), str(ids.device))

    def check(self, ids, pos, cp_size, kind, stripe_size, causal, window):
        """Raise ValueError unless the plan was made for this layout and mask."""
        meta = (tuple(ids.shape), int(cp_size), ra._kind_code(kind),
                int(stripe_size) if ra._kind_code(kind) == ra.STRIPED else 1,
                bool(causal), (int(window[0]), int(window[1])))
        if meta != self.meta:
            raise ValueError(f"ring plan made for {self.meta} (shape, shards, reorder, stripe, "
                             f"causal, window), used with {meta}")
        tok = self._token(ids, pos)
        if tok in self._seen:
            return
        if _layout_fingerprint(ids, pos) != self.fingerprint:
            raise ValueError("ring plan made for other segment ids / positions")
        self._seen.add(tok)

    def dim(self):
        return self.counts.dim()


def ring_plan(ids, pos, cp_size, kind="dual_chunk", stripe_size=1, *, num_q_heads, num_kv_heads,
              head_dim=128, dtype=torch.bfloat16, causal=True, window=(-1, -1), v_head_dim=None,
              halves=False):
    """The ring schedule of this segment layout: visible pairs of every ring
    step, ``counts int64 [R, R]`` on the host (rank, step), from the library's
    tile classification, wrapped in a :class:`RingPlan` that remembers the
    layout and mask it belongs to.

    The counts depend only on the segment ids and positions, so one plan
    serves every forward on the same layout.  A block with no visible pair
    contributes nothing to its rank's softmax ("Causal attention": such blocks
    are skipped), so :func:`ring_forward` given the plan runs only the steps
    with work and lets the last of them write the final output.

    ``halves`` (dual chunk): counts ``int64 [R, 2, R]`` (rank, stripe, step),
    each of the shard's two stripes apart; summed over the stripe axis they
    are the plain plan.  With it :func:`ring_forward` also finishes each
    stripe at its own last step with work.
    """
    b, t = ids.shape
    n = t // cp_size
    ids_r = ra.reorder(ids, cp_size, kind, stripe_size)
    pos_r = ra.reorder(pos, cp_size, kind, stripe_size)
    parts = [slice(0, n // 2), slice(n // 2, n)] if halves else [slice(0, n)]
    plan = torch.zeros((cp_size, len(parts), cp_size), dtype=torch.int64)
    for r in range(cp_size):
        for j, part in enumerate(parts):
            rows = slice(r * n + part.start, r * n + part.stop)
            for s in range(cp_size):
                c = (r - s) % cp_size
                cols = slice(c * n, (c + 1) * n)
                _, pairs = ra.classify_tiles(ids_r[:, rows], pos_r[:, rows], ids_r[:, cols],
                                             pos_r[:, cols], num_q_heads=num_q_heads,
                                             num_kv_heads=num_kv_heads, head_dim=head_dim,
                                             dtype=dtype, causal=causal, window=window,
                                             v_head_dim=v_head_dim)
                plan[r, j, s] = int(pairs.sum().item())
    return RingPlan(plan if halves else plan[:, 0], ids, pos, cp_size, kind, stripe_size, causal,
                    window)


def _stripe_schedule(hplan_r, cp_size):
    """Per ring step, the launches of one rank under a per-stripe plan
    ``[2, R]``: ``{(first, last): [stripes]}`` -- a stripe starts at its first
    step with work and finishes at its last (the last step if it has none)."""
    steps = [[s for s in range(cp_size) if int(hplan_r[j, s]) > 0] or [cp_size - 1]
             for j in (0, 1)]
    out = []
    for s in range(cp_size):
        roles = {}
        for j in (0, 1):
            if s in steps[j]:
                roles.setdefault((s == steps[j][0], s == steps[j][-1]), []).append(j)
        out.append(roles)
    return out


def needs_reordered_q(plan, cp_size):
    """False when a per-stripe plan ``[R, 2, R]`` never runs both stripes of a
    shard in one call: every call then reads one stripe, a contiguous range
    of the original sequence, and Q needs no reordered copy."""
    if isinstance(plan, RingPlan):
        plan = plan.counts
    if plan is None or plan.dim() != 3:
        return True
    return any(len(js) == 2 for r in range(cp_size)
               for roles in _stripe_schedule(plan[r], cp_size) for js in roles.values())


def _rank_steps_stripes(rank, cp_size, bufs, hplan, o, lse, scale, causal, window, step_hook,
                        q_orig=None, prep=None):
    """Rank ``rank``'s ring steps on a dual-chunk layout with a per-stripe plan
    ``hplan [2, R]``: each of the shard's two stripes starts at its first step
    with work and is finished (written to its original positions in ``o`` /
    ``lse``) at its last one, so a stripe with no work left costs nothing; at a
    step where both stripes play the same part one call covers them (a split
    output at the second stripe when that part is the last)."""
    t = bufs.q.shape[1]
    n = t // cp_size
    h = n // 2
    rows = slice(rank * n, (rank + 1) * n)
    q_r, id_r, pos_r = bufs.q[:, rows], bufs.ids[:, rows], bufs.pos[:, rows]
    halves = [slice(0, h), slice(h, n)]
    # the shard's stripes in the original order: stripe r, then stripe 2R-1-r
    orig = [slice(rank * h, (rank + 1) * h),
            slice((2 * cp_size - 1 - rank) * h, (2 * cp_size - rank) * h)]
    outs = [(o[:, orig[0]], lse[:, orig[0]]), (o[:, orig[1]], lse[:, orig[1]])]
    for s, roles in enumerate(_stripe_schedule(hplan, cp_size)):
        c = (rank - s) % cp_size
        cols = slice(c * n, (c + 1) * n)
        kv = (bufs.k[:, cols], bufs.v[:, cols])
        kmeta = (bufs.ids[:, cols], bufs.pos[:, cols])
        for (first, last), js in roles.items():
            qr = slice(0, n) if len(js) == 2 else halves[js[0]]
            # one stripe: its Q rows read in place from the original order
            qx = q_orig[:, orig[js[0]]] if q_orig is not None and len(js) == 1 else q_r[:, qr]
            args = (qx, *kv, id_r[:, qr], pos_r[:, qr], *kmeta)
            split = None
            if last and len(js) == 2:
                dst, dst_lse = outs[0]
                split = (h, outs[1][0], outs[1][1])
            elif last:
                dst, dst_lse = outs[js[0]]
            else:
                dst, dst_lse = bufs.acc[:, qr], bufs.acc_lse[:, qr]
            prepared, done = prep.get((rank, s, tuple(js)), c) if prep else (None, None)
            if step_hook:
                step_hook("attn_fwd", rank, s, True)
            if first:
                ra.attn_fwd(*args, scale=scale, causal=causal, window=window, out_dtype=dst.dtype,
                            out=dst, lse=dst_lse, workspace=bufs.workspace, split=split,
                            prepared=prepared)
            else:
                ra.attn_fwd_accumulate(*args, bufs.acc[:, qr], bufs.acc_lse[:, qr], scale=scale,
                                       causal=causal, window=window,
                                       out=None if not last else dst,
                                       lse=None if not last else dst_lse,
                                       workspace=bufs.workspace, split=split, prepared=prepared)
            if done:
                done()
            if step_hook:
                step_hook("attn_fwd", rank, s, False)


def ring_forward(q, k, v, ids, pos, cp_size, kind="dual_chunk", stripe_size=1, *, scale=None,
                 causal=True, window=(-1, -1), ranks=None, bufs: RingBuffers | None = None,
                 partial_dtype=torch.float32, out_dtype=None, step_hook=None, fused=True,
                 plan=None, fuse_inverse=True):
    """Ring-decomposed attention forward of self-attention inputs on one GPU.

    q ``[B,T,Hq,D]``, k/v ``[B,T,Hkv,D]``, ids/pos ``int32 [B,T]`` in the
    original token order.  Returns ``(o, lse)`` in the original order.  With
    ``ranks`` a subset of ranks, only those shards of the output are computed
    (the others are left as they were in ``bufs``).  With ``plan`` (from
    :func:`ring_plan` on the same layout and mask) the fused path runs only
    the steps whose blocks hold visible pairs; a per-stripe plan
    (``halves=True``) also lets each of a dual-chunk shard's two stripes stop
    at its own last step with work.

    With the dual-chunk reorder, the fused path and every rank run
    (``fuse_inverse``), the inverse reorder is folded into each rank's last
    step: a dual-chunk shard is two contiguous stripes of the original
    sequence (stripes r and 2R-1-r), so the last step writes its output with a
    split at the second stripe (``split`` of ``attn_fwd``), O and the LSE going
    straight to their original positions; no separate inverse-reorder pass is
    made.  The result is bit-identical.
    """
    if q.shape[1] != k.shape[1]:
        raise ValueError("the ring driver runs self-attention (Tq == Tk)")
    plan_obj = None
    if plan is not None:
        if not isinstance(plan, RingPlan):
            raise TypeError("plan must come from ring_plan()")
        plan.check(ids, pos, cp_size, kind, stripe_size, causal, window)
        plan_obj, plan = plan, plan.counts
    if bufs is None:
        bufs = RingBuffers.like(q, k, ids, cp_size, partial_dtype, out_dtype, v=v)
    b, t = ids.shape
    n = t // cp_size
    # every call of the ring reads at most a whole shard of queries against one chunk
    desc = ra.make_desc(b, n, n, q.shape[2], k.shape[2], q.shape[3], ra._dtype_code(q.dtype),
                        None, scale, causal, window, {"v_head_dim": v.shape[3]})
    prep = _Prepared(bufs, plan_obj, desc, (ra._dtype_code(q.dtype), q.shape[2], k.shape[2],
                                            q.shape[3], v.shape[3], bool(causal), tuple(window)))
    direct = (fuse_inverse and fused and ranks is None and cp_size > 1
              and ra._kind_code(kind) == ra.DUAL_CHUNK)
    # With a per-stripe plan whose calls each read one stripe, Q is read in
    # place (the reordered copy of Q is never made).
    q_in_place = direct and plan is not None and plan.dim() == 3 and not needs_reordered_q(
        plan, cp_size)
    if step_hook:
        step_hook("reorder", -1, -1, True)
    reorder_inputs(q, k, v, ids, pos, cp_size, kind, stripe_size, bufs, with_q=not q_in_place)
    if step_hook:
        step_hook("reorder", -1, -1, False)
    if direct:
        o = torch.empty_like(bufs.o)
        lse = torch.empty_like(bufs.lse)
    n = q.shape[1] // cp_size
    h = n // 2
    stripes = plan is not None and plan.dim() == 3
    if stripes and not direct:
        plan = plan.sum(1)          # per-stripe counts folded back into the plain plan
        stripes = False
    for r in (range(cp_size) if ranks is None else ranks):
        if stripes:
            _rank_steps_stripes(r, cp_size, bufs, plan[r], o, lse, scale, causal, window,
                                step_hook, q if q_in_place else None, prep)
            continue
        steps = None
        if plan is not None and fused:
            steps = [s for s in range(cp_size) if int(plan[r, s]) > 0] or [cp_size - 1]
        final = None
        if direct:
            # shard rows [0, h) are stripe r, rows [h, 2h) stripe 2R-1-r
            hi = slice((2 * cp_size - 1 - r) * h, (2 * cp_size - r) * h)
            final = (o[:, r * h:(r + 1) * h], lse[:, r * h:(r + 1) * h], (h, o[:, hi], lse[:, hi]))
        rank_steps(r, cp_size, bufs, scale=scale, causal=causal, window=window, step_hook=step_hook,
                   fused=fused, steps=steps, final=final, prep=prep)
    if direct:
        return o, lse
    if step_hook:
        step_hook("inverse_reorder", -1, -1, True)
    o = ra.inverse_reorder(bufs.o, cp_size, kind, stripe_size)
    lse = ra.inverse_reorder(bufs.lse, cp_size, kind, stripe_size)
    if step_hook:
        step_hook("inverse_reorder", -1, -1, False)
    return o, lse


class RingGraph:
    """One ring step (:func:`ring_forward` with a plan) captured as a HIP graph
    and replayed with a single launch.

    A ring step is a fixed sequence of library calls for a given segment
    layout, mask, shard count, reorder and shape: the reorders of K, V and the
    metadata, every attention call of every rank (each K/V chunk packed by
    its first call), and the inverse reorder folded into the last calls.  On
    small shards the step is bound by launching those calls one by one; a
    replay of the captured graph launches them all at once.

    The constructor copies ``q, k, v, ids, pos`` into tensors the graph owns,
    runs the step twice eagerly on a side stream (this allocates the driver's
    buffers and computes the plan's schedules, which the captured calls then
    reuse, so the graph holds no classification) and captures the third run.
    :meth:`replay` copies new Q, K, V values (same shapes and dtypes) into the
    graph's inputs, replays, and returns the graph's ``(o, lse)``: the same
    tensors every time, overwritten by each replay.  The segment ids and
    positions are fixed at capture, since the plan is tied to them.  The
    captured calls allocate nothing and clear nothing with a memset.
    """

    def __init__(self, q, k, v, ids, pos, cp_size, kind="dual_chunk", stripe_size=1, *, plan,
                 scale=None, causal=True, window=(-1, -1), partial_dtype=torch.float32,
                 out_dtype=None):
        if not isinstance(plan, RingPlan):
            raise TypeError("plan must come from ring_plan()")
        if not q.is_cuda:
            raise ValueError("RingGraph captures GPU work: q must be a device tensor")
        self.q, self.k, self.v = q.clone(), k.clone(), v.clone()
        self.ids, self.pos = ids.clone(), pos.clone()
        self.cp_size = cp_size
        self._kw = dict(kind=kind, stripe_size=stripe_size, scale=scale, causal=causal,
                        window=window, plan=plan, partial_dtype=partial_dtype,
                        out_dtype=out_dtype)
        self.bufs = RingBuffers.like(self.q, self.k, self.ids, cp_size, partial_dtype, out_dtype,
                                     v=self.v)
        dev = q.device
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(2):
                self._step()
        torch.cuda.current_stream(dev).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.o, self.lse = self._step()

    def _step(self):
        return ring_forward(self.q, self.k, self.v, self.ids, self.pos, self.cp_size,
                            bufs=self.bufs, **self._kw)

    def replay(self, q=None, k=None, v=None):
        """Copy the given inputs into the graph's own, replay, return ``(o, lse)``."""
        for name, dst, src in (("q", self.q, q), ("k", self.k, k), ("v", self.v, v)):
            if src is None:
                continue
            if src.shape != dst.shape or src.dtype != dst.dtype or src.device != dst.device:
                raise ValueError(f"{name}: expected {tuple(dst.shape)} {dst.dtype} on {dst.device}, "
                                 f"got {tuple(src.shape)} {src.dtype} on {src.device}")
            dst.copy_(src)
        self.graph.replay()
        return self.o, self.lse


def allgather_forward(q, k, v, ids, pos, cp_size, kind="striped", stripe_size=512, *, scale=None,
                      causal=True, window=(-1, -1), ranks=None, bufs: RingBuffers | None = None,
                      out_dtype=None, step_hook=None):
    """All-gather context-parallel forward of self-attention inputs on one GPU.

    The inputs are reordered (striped by default, as the tutorial's
    all-gather run with stripe_size 512), every rank's query shard attends to
    the full reordered K/V in one ``attn_fwd`` call, and O and the LSE are
    permuted back.  Shapes and return value as :func:`ring_forward`.
    """
    if q.shape[1] != k.shape[1]:
        raise ValueError("the all-gather driver runs self-attention (Tq == Tk)")
    b, t = ids.shape
    n = t // cp_size
    if bufs is None:
        bufs = RingBuffers.like(q, k, ids, cp_size, out_dtype=out_dtype, partials=False, v=v)
    desc = ra.make_desc(b, n, t, q.shape[2], k.shape[2], q.shape[3], ra._dtype_code(q.dtype),
                        None, scale, causal, window, {"v_head_dim": v.shape[3]})
    # the whole K/V is packed once, by the first shard's call
    prep = _Prepared(bufs, None, desc, None)
    if step_hook:
        step_hook("reorder", -1, -1, True)
    reorder_inputs(q, k, v, ids, pos, cp_size, kind, stripe_size, bufs)
    if step_hook:
        step_hook("reorder", -1, -1, False)
    for r in (range(cp_size) if ranks is None else ranks):
        rows = slice(r * n, (r + 1) * n)
        if step_hook:
            step_hook("attn_fwd", r, 0, True)
        prepared, done = prep.get(None, 0)
        ra.attn_fwd(bufs.q[:, rows], bufs.k, bufs.v, bufs.ids[:, rows], bufs.pos[:, rows],
                    bufs.ids, bufs.pos, scale=scale, causal=causal, window=window,
                    out_dtype=bufs.o.dtype, out=bufs.o[:, rows], lse=bufs.lse[:, rows],
                    prepared=prepared)
        done()
        if step_hook:
            step_hook("attn_fwd", r, 0, False)
    if step_hook:
        step_hook("inverse_reorder", -1, -1, True)
    o = ra.inverse_reorder(bufs.o, cp_size, kind, stripe_size)
    lse = ra.inverse_reorder(bufs.lse, cp_size, kind, stripe_size)
    if step_hook:
        step_hook("inverse_reorder", -1, -1, False)
    return o, lse
