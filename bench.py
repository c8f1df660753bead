"""Benchmark: attention forward TFLOP/s on visible (query, key) pairs, one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  For the default workload (one device's share of the
TransformerEngine tutorial's long-context case, run as a 4-shard ring) that is:
causal load-balancing reorder of K, V, segment ids and positions (Q is read in
place); for each of the 4 shards, its ring steps -- attn_fwd for the first
block with visible pairs, then attn_fwd_accumulate for the next ones, each
folding its block into the running fp32 partial in its epilogue (the merge of
the ring update, fused; ``--unfused`` runs attn_fwd + attn_merge instead);
inverse reorder of O and LSE, folded into the forward's stores (a dual-chunk
shard is two contiguous stripes of the sequence, written with a split output
at their original positions).  A plan computed once per layout skips the ring
steps whose blocks hold no visible pair and finishes each stripe at its own
last step with work (``--plan-by-rank``, ``--no-plan`` for the coarser
schedules).  ``--ring-layout striped`` runs the tutorial's ring layout
(striped, stripe 1) instead of the dual-chunk one.  All four shards are
computed, so a step is the complete forward of B=2 x 65536 tokens; FLOPs count
only visible pairs (2 * (D + Dv) * Hq per pair).

Prints one JSON line.  ``roofline`` is measured live with HIP events that the
library records on its stream right before and after the attention kernel of
every forward call (``ra_profile_next_kernel``; the call's tile classification
and K/V repack fall outside); ``cpu_baseline`` times the fp64 oracle on a
bounded row sample of the same inputs over a process pool of the host's
cores.  ``detail`` also carries, measured in the same process: the other
workloads (packed GQA and sliding-window single calls, the sharded packed
workload's 4 x (attn_fwd + attn_merge) pipeline, the long-context ring under
the other layout), one backward call on a long-context all-gather shard, the
merge and reorder kernels on their own, and the ring plan's cost.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import blockwise_online_softmax_fwd_amd as bosf  # noqa: E402
from workloads import get, packed_metadata  # noqa: E402

METRIC = "attention fwd TFLOP/s (visible pairs) + % of bf16 MFMA peak, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3          # MI355X fp32 matrix (and vector) peak: 256 CUs x 4 SIMDs x 64 flops/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_inputs(w, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shp_q = (w.batch, w.seq_len, w.num_q_heads, w.head_dim)
    shp_kv = (w.batch, w.seq_len, w.num_kv_heads, w.head_dim)
    q = torch.randn(shp_q, generator=g, device=dev).to(dt)
    k = torch.randn(shp_kv, generator=g, device=dev).to(dt)
    v = torch.randn(shp_kv[:3] + (w.dv,), generator=g, device=dev).to(dt)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    return q, k, v, ids.to(dev), pos.to(dev)


def fwd_flops(w, pairs):
    """2*D flops for Q K^T and 2*Dv for P V per visible pair and query head."""
    return 2.0 * (w.head_dim + w.dv) * w.num_q_heads * pairs


def visible_pairs(w, ids, pos, dtype):
    """Visible pairs of the unsplit problem, by the library's classification."""
    _, pairs = bosf.classify_tiles(ids, pos, ids, pos, num_q_heads=w.num_q_heads,
                                   num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                   v_head_dim=w.dv, dtype=dtype, causal=w.causal,
                                   window=w.window)
    return int(pairs.sum().item())


class EventLog:
    """Event pairs around library calls, grouped by call name."""

    def __init__(self):
        self.open = {}
        self.done = {}
        self.enabled = False

    def hook(self, name, rank, step, begin):
        if not self.enabled:
            return
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        if begin:
            self.open[name] = ev
            if name == "attn_fwd":
                # the attention kernel alone, recorded by the library itself
                pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                bosf.profile_next_kernel(*pair)
                self.open["attn_kernel"] = pair
        else:
            self.done.setdefault(name, []).append((self.open.pop(name), ev, rank))
            if name == "attn_fwd":
                self.done.setdefault("attn_kernel", []).append(self.open.pop("attn_kernel")
                                                               + (rank,))

    def ms(self, name):
        return [a.elapsed_time(b) for a, b, _ in self.done.get(name, [])]

    def ranks(self, name):
        return [r for _, _, r in self.done.get(name, [])]


def timed(fn, warmup, iters):
    """Per-call milliseconds of ``fn`` (events on the current stream)."""
    for _ in range(warmup):
        fn()
    evs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def measured_traffic(launches_per_step):
    """HBM bytes per attn_fwd launch from the committed rocprofv3 counter runs.

    ``profiles/attn_fwd_longctx_ring4_traffic.json`` records FETCH_SIZE and
    WRITE_SIZE summed over the forward's launches of one step, already scaled
    by the factors a plain copy kernel of known size gave, together with the
    SHA-256 of the forward kernel's source at the time and the number of
    launches per step; if the kernel or the launch structure has changed
    since, the figure no longer applies and None is returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fwd_longctx_ring4_traffic.json")
    src = os.path.join(ROOT, "blockwise_online_softmax_fwd_amd", "csrc", "attn_bf16.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha or rec.get("launches_per_step") != launches_per_step:
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------------------- forward step

def run_forward(w, dev, inputs, *, steps, warmup, strategy="ring", unfused=False,
                separate_inverse=False, plan_mode="stripes"):
    """Time ``steps`` forward steps of workload ``w`` (after ``warmup``).

    strategy "ring" (sharded workloads: ring steps with partials, merges fused
    unless ``unfused``), "allgather" (each shard against the whole K/V in one
    call) or "single" (one unsplit call).  plan_mode "stripes" (per-stripe
    plan on a dual-chunk layout, per rank otherwise), "rank" or "none".
    Returns a dict of the measurements."""
    q, k, v, ids, pos = inputs
    visible = visible_pairs(w, ids, pos, q.dtype)
    flops = fwd_flops(w, visible)
    ev = EventLog()
    out = {}
    plan = None
    plan_ms = None
    if strategy == "allgather":
        bufs = bosf.RingBuffers.like(q, k, ids, w.cp_size, partials=False, v=v)

        def step():
            out.clear()   # the previous step's output is not held across the next
            out["o"], out["lse"] = bosf.allgather_forward(
                q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, causal=w.causal,
                window=w.window, bufs=bufs, step_hook=ev.hook)
    elif w.cp_size > 1:
        bufs = bosf.RingBuffers.like(q, k, ids, w.cp_size, v=v)
        # The ring schedule of this segment layout (visible pairs per rank,
        # dual-chunk stripe and step), computed once outside the timed region
        # like the layout itself; steps whose blocks hold no visible pair are
        # then not launched, and each stripe is finished at its own last step
        # with work.
        if plan_mode != "none" and not unfused:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            plan = bosf.ring_plan(ids, pos, w.cp_size, w.reorder, w.stripe,
                                  num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                                  head_dim=w.head_dim, dtype=q.dtype, causal=w.causal,
                                  window=w.window, v_head_dim=w.dv,
                                  halves=w.reorder == "dual_chunk" and plan_mode == "stripes")
            plan_ms = (time.perf_counter() - t0) * 1000.0
            log(f"ring plan ({plan_ms:.1f} ms; visible pairs per rank x step): "
                f"{plan.counts.tolist()}")

        def step():
            out.clear()
            out["o"], out["lse"] = bosf.ring_forward(
                q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, causal=w.causal,
                window=w.window, bufs=bufs, step_hook=ev.hook, fused=not unfused, plan=plan,
                fuse_inverse=not separate_inverse)
    else:
        bufs = None
        o = torch.empty(q.shape[:3] + (w.dv,), dtype=q.dtype, device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        desc = bosf.make_desc(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                              w.head_dim, 0 if w.dtype == "bf16" else 1,
                              strides={"v_head_dim": w.dv})
        wsp = torch.empty(bosf.workspace_size(desc), dtype=torch.uint8, device=dev)

        def step():
            ev.hook("attn_fwd", 0, 0, True)
            bosf.attn_fwd(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window, out=o,
                          lse=lse, workspace=wsp)
            ev.hook("attn_fwd", 0, 0, False)
            out["o"], out["lse"] = o, lse

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev.enabled = True
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev.enabled = False
    ms_step = (t1 - t0) * 1000.0 / steps
    kern_ms = ev.ms("attn_kernel")
    attn_ms = ev.ms("attn_fwd")
    per_step = len(kern_ms) // steps
    step_kern = [sum(kern_ms[i * per_step:(i + 1) * per_step]) for i in range(steps)]
    return {"w": w, "visible": visible, "flops": flops, "ms_step": ms_step,
            "value": flops / (ms_step / 1000.0) / 1e12, "ev": ev, "kern_ms": kern_ms,
            "attn_ms": attn_ms, "per_step": per_step, "step_kern": step_kern, "plan": plan,
            "plan_ms": plan_ms, "out": out, "bufs": bufs, "steps": steps}


def forward_summary(res):
    """Kernel-time figures of a :func:`run_forward` result."""
    steps, flops = res["steps"], res["flops"]
    kern_total = float(sum(res["kern_ms"]))
    attn_total = float(sum(res["attn_ms"]))
    n = len(res["kern_ms"])
    achieved = flops * steps / (kern_total / 1000.0) / 1e12
    median_kern = float(np.median(res["step_kern"]))
    return {"ms_per_step": res["ms_step"], "TFLOPs": res["value"],
            "visible_pairs_per_step": res["visible"],
            "attn_fwd_launches_per_step": res["per_step"],
            "attn_kernel_ms_per_step": kern_total / steps,
            "attn_kernel_ms_per_step_median": median_kern,
            "attn_kernel_ms_per_step_min": float(min(res["step_kern"])),
            "attn_kernel_avg_ms_per_launch": kern_total / n,
            "attn_kernel_TFLOPs": achieved,
            "attn_kernel_TFLOPs_median": flops / (median_kern / 1000.0) / 1e12,
            "attn_kernel_frac_of_peak": achieved / PEAK_BF16_TFLOPS,
            "attn_fwd_call_ms_per_step": attn_total / steps,
            "call_TFLOPs_incl_classify_pack": flops * steps / (attn_total / 1000.0) / 1e12}


# ----------------------------------------------------------------------------- other measurements

def single_call(w, dev, warmup=2, iters=10):
    """One attn_fwd over a whole unsplit workload: call and kernel times; the
    kernel's rate against the matrix peak of its input type (bf16 or fp32)."""
    q, k, v, ids, pos = make_inputs(w, dev)
    visible = visible_pairs(w, ids, pos, q.dtype)
    flops = fwd_flops(w, visible)
    o = torch.empty(q.shape[:3] + (w.dv,), dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    desc = bosf.make_desc(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, 0 if w.dtype == "bf16" else 1, strides={"v_head_dim": w.dv})
    wsp = torch.empty(bosf.workspace_size(desc), dtype=torch.uint8, device=dev)
    kev = []

    def call():
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        bosf.profile_next_kernel(*pair)
        kev.append(pair)
        bosf.attn_fwd(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window, out=o,
                      lse=lse, workspace=wsp)

    call_ms = timed(call, warmup, iters)
    kern_ms = [a.elapsed_time(b) for a, b in kev[warmup:]]
    km = float(np.median(kern_ms))
    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    return {"workload": f"{w.name}: {w.describe()}", "visible_pairs": visible, "flops": flops,
            "call_ms_median": float(np.median(call_ms)), "call_ms_min": float(min(call_ms)),
            "kernel_ms_median": km, "kernel_ms_min": float(min(kern_ms)),
            "kernel_TFLOPs": flops / (km / 1000.0) / 1e12,
            "bound": "mfma", "peak_TFLOPs": peak,
            "kernel_frac_of_peak": flops / (km / 1000.0) / 1e12 / peak,
            "call_TFLOPs": flops / (float(np.median(call_ms)) / 1000.0) / 1e12}


def graph_ring(w, dev, inputs, steps=10, warmup=2):
    """The fused, planned ring step of workload ``w`` captured once as a HIP
    graph (``RingGraph``) and replayed: wall time per replay over ``steps``
    replays bracketed by synchronisations, and whether the first replay's
    output equals the eager driver's bit for bit."""
    q, k, v, ids, pos = inputs
    visible = visible_pairs(w, ids, pos, q.dtype)
    flops = fwd_flops(w, visible)
    plan = bosf.ring_plan(ids, pos, w.cp_size, w.reorder, w.stripe, num_q_heads=w.num_q_heads,
                          num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, dtype=q.dtype,
                          causal=w.causal, window=w.window, v_head_dim=w.dv,
                          halves=w.reorder == "dual_chunk")
    t0 = time.perf_counter()
    graph = bosf.RingGraph(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, plan=plan,
                           causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    capture_ms = (time.perf_counter() - t0) * 1000.0
    o_e, l_e = bosf.ring_forward(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, plan=plan,
                                 causal=w.causal, window=w.window)
    o_g, l_g = graph.replay()
    same = bool(torch.equal(o_e, o_g) and torch.equal(l_e, l_g))
    del o_e, l_e
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    del graph
    return {"ms_per_step": ms, "TFLOPs": flops / (ms / 1000.0) / 1e12,
            "capture_ms_incl_two_eager_steps": capture_ms, "first_replay_equals_eager": same,
            "note": "one replay = the whole ring step (reorders, every attention call, folded "
                    "inverse reorder) launched from a captured HIP graph"}


def ring_pipeline(w, dev, steps=10, warmup=2):
    """The sharded workload as 4 shards x (4 attn_fwd + 3 attn_merge), every
    ring step launched (no plan), plus the fused, planned ring of the
    headline path on the same inputs, launched call by call and replayed from
    a captured HIP graph."""
    inputs = make_inputs(w, dev)
    res = {}
    for name, kw in (("unfused_4fwd_3merge", dict(unfused=True, plan_mode="none")),
                     ("fused_planned", dict())):
        r = run_forward(w, dev, inputs, steps=steps, warmup=warmup, **kw)
        s = forward_summary(r)
        merges = r["ev"].ms("attn_merge")
        if merges:
            s["attn_merge_ms_per_step"] = sum(merges) / steps
            s["attn_merge_calls_per_step"] = len(merges) // steps
            s["pipeline_ms_per_step_fwd_calls_plus_merges"] = (
                s["attn_fwd_call_ms_per_step"] + s["attn_merge_ms_per_step"])
        s["step_reorder_ms"] = sum(r["ev"].ms("reorder")) / steps
        s["step_inverse_reorder_ms"] = sum(r["ev"].ms("inverse_reorder")) / steps
        res[name] = s
    res["fused_planned_graph_replay"] = graph_ring(w, dev, inputs, steps=steps, warmup=warmup)
    res["workload"] = f"{w.name}: {w.describe()}"
    return res


def backward_shard(w, dev, stripe=512, warmup=1, iters=3):
    """One attn_bwd call on shard 0 of the all-gather layout (striped by
    ``stripe``): its queries against the whole K/V, fp32 gradients."""
    w = dataclasses.replace(w, reorder="striped", stripe=stripe)
    q, k, v, ids, pos = make_inputs(w, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 17)
    cp = w.cp_size
    q, k, v, ids, pos = (bosf.reorder(t, cp, "striped", stripe) for t in (q, k, v, ids, pos))
    n = w.seq_len // cp
    qs = q[:, :n].contiguous()
    del q
    do = torch.randn(qs.shape[:3] + (w.dv,), generator=g, device=dev).to(torch.bfloat16)
    iq, pq = ids[:, :n], pos[:, :n]
    o, lse = bosf.attn_fwd(qs, k, v, iq, pq, ids, pos, causal=w.causal, window=w.window)
    _, pairs = bosf.classify_tiles(iq, pq, ids, pos, num_q_heads=w.num_q_heads,
                                   num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                   v_head_dim=w.dv, causal=w.causal, window=w.window)
    visible = int(pairs.sum().item())
    flops = 2.0 * (3 * w.head_dim + 2 * w.dv) * w.num_q_heads * visible
    grads = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in (qs, k, v)]
    desc = bosf.make_desc(w.batch, n, w.seq_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                          strides={"q_meta_batch_stride": ids.stride(0), "v_head_dim": w.dv})
    wsp = torch.empty(bosf.bwd_workspace_size(desc), dtype=torch.uint8, device=dev)

    def call():
        bosf.attn_bwd(qs, k, v, iq, pq, ids, pos, o, lse, do, causal=w.causal, window=w.window,
                      dq=grads[0], dk=grads[1], dv=grads[2], workspace=wsp)

    ms = timed(call, warmup, iters)
    m = float(np.median(ms))
    return {"workload": f"{w.name} backward, all-gather shard 0 of 4 (striped {stripe}): "
                        f"{n} queries per row against all {w.seq_len} keys, fp32 gradients",
            "visible_pairs": visible, "flops": flops, "flops_per_pair": "2*(3D+2Dv)*Hq",
            "call_ms_median": m, "call_ms_min": float(min(ms)),
            "TFLOPs": flops / (m / 1000.0) / 1e12,
            "frac_of_peak": flops / (m / 1000.0) / 1e12 / PEAK_BF16_TFLOPS}


def standalone_rates(w, dev, out, inputs):
    """attn_merge and both reorders on their own at the long-context step's
    shapes (outside the step), as HBM rates."""
    q, k, v, ids, pos = inputs
    b, t, hq, d = q.shape
    n = t // w.cp_size
    det = {}
    # inverse reorder of the step's O and LSE (8.6 GB moved)
    o_s, l_s = out["o"], out["lse"]

    def inv():
        bosf.inverse_reorder(o_s, w.cp_size, w.reorder, w.stripe)
        bosf.inverse_reorder(l_s, w.cp_size, w.reorder, w.stripe)
    ims = float(np.median(timed(inv, 2, 5)))
    inv_bytes = 2 * (o_s.numel() * o_s.element_size() + l_s.numel() * 4)
    det.update({"inverse_reorder_standalone_ms": ims, "inverse_reorder_standalone_bytes": inv_bytes,
                "inverse_reorder_standalone_GBs": inv_bytes / (ims / 1000.0) / 1e9})
    # forward reorder of Q, K, V, ids and positions (9.7 GB moved)
    dst = [torch.empty_like(x) for x in inputs]

    def fwd():
        for x, y in zip(inputs, dst):
            bosf.reorder(x, w.cp_size, w.reorder, w.stripe, out=y)
    fms = float(np.median(timed(fwd, 2, 5)))
    f_bytes = 2 * sum(x.numel() * x.element_size() for x in inputs)
    det.update({"reorder_standalone_ms": fms, "reorder_standalone_bytes": f_bytes,
                "reorder_standalone_GBs": f_bytes / (fms / 1000.0) / 1e9})
    del dst
    # attn_merge: two fp32 shard partials with finite LSE (every row reads both
    # operands): 3 * D * 4 + 12 bytes per (b, t, h) row
    pa = torch.randn((b, n, hq, d), device=dev)
    pb = torch.randn_like(pa)
    la = torch.randn((b, n, hq), device=dev)
    lb = torch.randn_like(la)
    outm = torch.empty_like(pa)
    outl = torch.empty_like(la)
    mms = float(np.median(timed(lambda: bosf.attn_merge(pa, la, pb, lb, out=outm, lse_out=outl),
                                2, 5)))
    mbytes = b * n * hq * (3 * 4 * d + 12)
    det.update({"attn_merge_ms_per_call": mms, "attn_merge_bytes_per_call": mbytes,
                "attn_merge_GBs": mbytes / (mms / 1000.0) / 1e9})
    return det


# ----------------------------------------------------------------------------- CPU baseline

def _host_info(workers):
    from oracle.pool import cpu_model
    return {"cores": int(workers), "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "threads_per_worker": 1}


def cpu_baseline(w, q, k, v, ids, pos, budget_s, o=None, lse=None):
    """The fp64 oracle (``oracle.attention_rows``' row function) on a bounded
    random sample of valid query rows of the same inputs, all heads, spread
    over a process pool of the host's cores (one BLAS thread each).  The rate
    counts the sample's visible pairs over the time of the timed rounds;
    starting the pool and staging K/V for it are reported apart (``setup_s``).

    With the step's output (``o``, ``lse`` in token order), the oracle rows are
    also compared with the GPU's: returns the baseline and the sample's max |O|
    and |LSE| differences and -inf mismatch count (or None)."""
    import oracle
    from oracle.pool import RowPool, pool_workers
    idc, posc = ids.cpu(), pos.cpu()
    rng = np.random.default_rng(0)
    valid = np.argwhere(idc.numpy() != 0)
    order = [tuple(int(x) for x in valid[j]) for j in rng.permutation(len(valid))]
    workers = pool_workers()
    scale = w.head_dim ** -0.5
    rows, refs, pairs = [], [], 0
    t_setup = time.perf_counter()
    with RowPool(k, v, idc, posc, idc, posc, workers) as pool:
        batch = 2 * workers

        def round_(sel):
            bi = torch.tensor([r[0] for r in sel], device=q.device)
            ti = torch.tensor([r[1] for r in sel], device=q.device)
            qr = q[bi, ti].to("cpu", torch.float64).numpy()
            return pool.forward(qr, sel, scale=scale, causal=w.causal, window=w.window)

        # the first round starts the workers; it is checked below but not timed
        warm = order[:workers]
        wo, wl = round_(warm)
        setup_s = time.perf_counter() - t_setup
        pos_i = workers
        t0 = time.perf_counter()
        while pos_i < len(order) and time.perf_counter() - t0 < budget_s:
            sel = order[pos_i:pos_i + batch]
            pos_i += len(sel)
            refs.append(round_(sel))
            rows += sel
        dt = time.perf_counter() - t0
    for b, i in rows:
        pairs += int(oracle.visible(idc[b, i:i + 1], posc[b, i:i + 1], idc[b], posc[b],
                                    w.causal, w.window).sum())
    flops = fwd_flops(w, pairs)
    base = {"value": flops / dt / 1e12 if dt > 0 else 0.0, "unit": "TFLOP/s", "kind": "oracle",
            **_host_info(workers),
            "sample": f"{len(rows)} random valid query rows x all {w.num_q_heads} heads "
                      f"({pairs} visible pairs, {flops / 1e9:.1f} GFLOP fp64) in {dt:.1f} s "
                      f"over {workers} worker processes",
            "setup_s": setup_s}
    check = None
    all_rows = warm + rows
    if o is not None and all_rows:
        all_o = np.concatenate([wo] + [r[0] for r in refs])
        all_l = np.concatenate([wl] + [r[1] for r in refs])
        bi = torch.tensor([r[0] for r in all_rows], device=o.device)
        ti = torch.tensor([r[1] for r in all_rows], device=o.device)
        go = o[bi, ti].to("cpu", torch.float64).numpy()
        gl = lse[bi, ti].to("cpu", torch.float64).numpy()
        ei, er = np.isneginf(gl), np.isneginf(all_l)
        live = ~(ei | er)
        check = {"rows": len(all_rows), "heads": w.num_q_heads,
                 "max_abs_o": float(np.abs(go - all_o).max()),
                 "max_abs_lse": float(np.abs(gl[live] - all_l[live]).max()) if live.any() else 0.0,
                 "lse_neg_inf_mismatches": int((ei != er).sum())}
    return base, check


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=5, help="workload number (1-6)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads, the backward call and the standalone "
                         "merge/reorder rates in detail")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other workloads and the backward call (keep the standalone "
                         "merge/reorder rates)")
    ap.add_argument("--unfused", action="store_true",
                    help="ring steps write separate partials folded by attn_merge")
    ap.add_argument("--separate-inverse", action="store_true",
                    help="ring: run the inverse reorder of O and LSE as its own pass instead of "
                         "folding it into each rank's last ring step")
    ap.add_argument("--plan-by-rank", action="store_true",
                    help="ring: plan steps per rank only (both stripes of a shard finish at the "
                         "rank's last step with work)")
    ap.add_argument("--no-plan", action="store_true",
                    help="launch every ring step, also those whose blocks hold no visible pair")
    ap.add_argument("--ring-layout", choices=("dual_chunk", "striped"), default=None,
                    help="load-balancing layout of the ring (default: the workload's, dual "
                         "chunk; striped uses stripe 1, the tutorial's ring layout)")
    ap.add_argument("--strategy", choices=("ring", "allgather"), default="ring",
                    help="context-parallel strategy of the sharded workloads: ring steps with "
                         "partials, or each shard against the whole gathered K/V (striped)")
    ap.add_argument("--stripe", type=int, default=512,
                    help="stripe size of the all-gather strategy's striped reorder")
    ap.add_argument("--backward", action="store_true",
                    help="time the attention backward (attn_bwd) instead of the forward: every "
                         "shard of the all-gather strategy against the whole K/V, o and lse from "
                         "the forward computed once outside the timed region")
    ap.add_argument("--grad-dtype", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB with a plain device copy kernel "
                         "(a known-size reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the ring is "
              "emulated shard by shard on a single device", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = get(args.workload)
    allgather = args.strategy == "allgather" and w.cp_size > 1
    if allgather:
        w = dataclasses.replace(w, reorder="striped", stripe=args.stripe)
    elif args.ring_layout == "striped" and w.cp_size > 1:
        w = dataclasses.replace(w, reorder="striped", stripe=1)
    bosf.load_library()
    if args.backward:
        return bench_backward(args, w, dev)
    desc = w.describe()
    if allgather:
        desc = desc.replace(f"{w.cp_size} shards x {w.cp_size} ring steps",
                            f"{w.cp_size} shards (stripe {w.stripe}), each against the whole "
                            "gathered K/V in one call")
    elif w.reorder == "striped":
        desc = desc.replace("striped reorder", f"striped({w.stripe}) reorder")
    log(f"workload {w.cfg} {w.name}: {desc}")
    inputs = make_inputs(w, dev)
    q, k, v, ids, pos = inputs
    plan_mode = "none" if args.no_plan else ("rank" if args.plan_by_rank else "stripes")
    strategy = "allgather" if allgather else ("ring" if w.cp_size > 1 else "single")
    res = run_forward(w, dev, inputs, steps=args.steps, warmup=args.warmup, strategy=strategy,
                      unfused=args.unfused, separate_inverse=args.separate_inverse,
                      plan_mode=plan_mode)
    value, ms_step, flops = res["value"], res["ms_step"], res["flops"]
    log(f"visible pairs {res['visible']}, {flops / 1e12:.3f} TFLOP per step; "
        f"{ms_step:.3f} ms/step, {value:.1f} TFLOP/s")
    summ = forward_summary(res)
    achieved = summ["attn_kernel_TFLOPs"]
    per_step = res["per_step"]
    plan = res["plan"]
    detail = {k_: v_ for k_, v_ in summ.items() if k_ not in ("ms_per_step", "TFLOPs")}
    detail["pct_of_bf16_peak_whole_step"] = 100.0 * value / PEAK_BF16_TFLOPS
    if res["plan_ms"] is not None:
        detail["ring_plan_ms"] = res["plan_ms"]
        detail["ring_plan_note"] = ("once per segment layout, outside the timed region: "
                                    "classification of every (rank, stripe, step) block")
    if w.cp_size > 1:
        # per rank: the attention kernel time of its share per step and, with
        # the ring plan's pair counts, its own rate (the headline aggregates
        # all ranks' flops over their summed kernel time)
        ev = res["ev"]
        kern_ms = res["kern_ms"]
        rk = ev.ranks("attn_kernel")
        rank_ms = [sum(m for m, r in zip(kern_ms, rk) if r == rr) / args.steps
                   for rr in range(w.cp_size)]
        detail["attn_kernel_ms_per_step_by_rank"] = rank_ms
        if not allgather and plan is not None:
            rank_tf = [fwd_flops(w, float(plan.counts[rr].sum())) / (rank_ms[rr] / 1000.0) / 1e12
                       for rr in range(w.cp_size)]
            detail["attn_kernel_TFLOPs_by_rank"] = rank_tf
            detail["attn_kernel_TFLOPs_min_rank"] = min(rank_tf)
        # Q is read in place (no reordered copy) when the per-stripe plan never
        # runs both stripes of a shard in one call
        q_moved = (allgather or args.unfused or args.separate_inverse or plan is None
                   or bosf.needs_reordered_q(plan, w.cp_size))
        detail["q_reordered"] = bool(q_moved)
        reorder_ms = sum(ev.ms("reorder")) / args.steps
        fwd_bytes = 2 * ((q.numel() * 2 if q_moved else 0) + k.numel() * 2 + v.numel() * 2
                         + 2 * ids.numel() * 4)
        detail.update({
            "strategy": ("all-gather: each shard against the whole K/V, no merge" if allgather
                         else "ring: unfused, attn_merge per step" if args.unfused
                         else "ring: merges fused into attn_fwd_accumulate epilogues, "
                              + ("every step launched" if args.no_plan
                                 else "steps without visible pairs skipped")),
            "step_reorder_ms": reorder_ms,
            "step_reorder_bytes": fwd_bytes,
            "step_reorder_GBs": fwd_bytes / (reorder_ms / 1000.0) / 1e9,
            "step_reorder_note": ("the in-step reorder moves K, V, ids and positions only when Q "
                                  "is read in place (about 1.1 GB, partly cache-resident); the "
                                  "standalone reorder of all five tensors is the HBM rate"),
        })
        inv_ms = ev.ms("inverse_reorder")
        if inv_ms:
            inv_bytes = 2 * (res["out"]["o"].numel() * 2 + res["out"]["lse"].numel() * 4)
            inv_step = sum(inv_ms) / args.steps
            detail.update({"step_inverse_reorder_ms": inv_step,
                           "step_inverse_reorder_GBs": inv_bytes / (inv_step / 1000.0) / 1e9})
        else:
            detail["inverse_reorder"] = ("folded into the forward's stores: each dual-chunk "
                                         "stripe's O and LSE are written at their original "
                                         "positions (split output)")
        if args.unfused:
            detail["attn_merge_ms_per_step"] = sum(ev.ms("attn_merge")) / args.steps
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": (measured_traffic(per_step) if args.workload == 5 and not allgather
                            and w.reorder == "dual_chunk" and not args.unfused
                            and not args.no_plan and not args.plan_by_rank else None),
                "kernel": "attn_fwd_bf16_kernel (events recorded by the library around the "
                          "kernel alone)",
                "per_launch_flops": flops * args.steps / len(res["kern_ms"])}

    out = res["out"]
    if not args.no_extra and w.cp_size > 1 and not allgather:
        log("standalone merge and reorder rates")
        detail.update(standalone_rates(w, dev, out, inputs))

    if args.copy_probe_mib > 0:
        n_el = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n_el, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        detail["copy_probe_bytes_each_way"] = n_el * 4
        del src, dst

    cpu = check = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a host row sample")
        cpu, check = cpu_baseline(w, q, k, v, ids, pos, args.cpu_seconds, out.get("o"),
                                  out.get("lse"))
        log(f"cpu baseline {cpu['value'] * 1000:.2f} GFLOP/s on {cpu['cores']} cores")

    if not args.no_extra and not args.no_other_configs and args.workload == 5 and not allgather:
        # the other configurations, measured in this same process
        res["bufs"] = None
        out.clear()
        del q, k, v, ids, pos, inputs, res
        torch.cuda.empty_cache()
        other = {}
        other_kind = "striped" if w.reorder == "dual_chunk" else "dual_chunk"
        w5 = dataclasses.replace(get(5), reorder=other_kind, stripe=1)
        log(f"workload 5 under the {other_kind} ring layout")
        r5 = run_forward(w5, dev, make_inputs(w5, dev), steps=5, warmup=2,
                         plan_mode="stripes" if other_kind == "dual_chunk" else "rank")
        s5 = forward_summary(r5)
        s5["workload"] = (f"{w5.name}: "
                          + w5.describe().replace("striped reorder", "striped(1) reorder"))
        s5["ring_plan_ms"] = r5["plan_ms"]
        other[f"w5_ring_{other_kind}{'1' if other_kind == 'striped' else ''}"] = s5
        del r5
        torch.cuda.empty_cache()
        log("workload 5 ring step replayed from a captured HIP graph")
        other["w5_ring_graph_replay"] = graph_ring(get(5), dev, make_inputs(get(5), dev),
                                                   steps=5, warmup=2)
        torch.cuda.empty_cache()
        for cfg in (1, 2, 4, 6):
            log(f"workload {cfg} (one call)")
            other[f"w{cfg}_single_call"] = single_call(get(cfg), dev)
            torch.cuda.empty_cache()
        # the fp32 path (vector unit) at the sliding-window workload's shape
        w4f = dataclasses.replace(get(4), dtype="f32", name="causal_swa4096_gqa_f32")
        log("workload 4's shape in fp32 (one call)")
        other["w4_shape_f32_single_call"] = single_call(w4f, dev, warmup=1, iters=3)
        torch.cuda.empty_cache()
        log("workload 3 ring pipeline")
        other["w3_ring_pipeline"] = ring_pipeline(get(3), dev)
        torch.cuda.empty_cache()
        log("one backward call on a workload 5 all-gather shard")
        other["w5_backward_allgather_shard"] = backward_shard(get(5), dev)
        torch.cuda.empty_cache()
        detail["other_configs"] = other

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "config": {"workload": f"{w.name}{' all-gather' if allgather else ''}: {desc}",
                   "batch": w.batch,
                   "seq_len": w.seq_len, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "v_head_dim": w.dv,
                   "window": list(w.window), "cp_shards": w.cp_size, "reorder": w.reorder,
                   "stripe": w.stripe, "strategy": "allgather" if allgather else "ring"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sample_parity": check,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_bwd(w, q, k, v, do, q_ids, q_pos, kv_ids, kv_pos, budget_s, dq=None):
    """Backward oracle (fp64, host) on a bounded random sample of one shard's
    query rows over a process pool of the host's cores: dQ of each row over
    all heads (products S, dP, dQ: 2*(2D+Dv)*Hq flops per visible pair, 6*D*Hq
    when D = Dv).  With the shard's dQ from the GPU, the sampled rows are also
    compared: relative Frobenius error and max error over max |dQ| of the
    sample (or None)."""
    import oracle
    from oracle.pool import RowPool, pool_workers
    iq, pq, ik, pk = q_ids.cpu(), q_pos.cpu(), kv_ids.cpu(), kv_pos.cpu()
    rng = np.random.default_rng(1)
    valid = np.argwhere(iq.numpy() != 0)
    order = [tuple(int(x) for x in valid[j]) for j in rng.permutation(len(valid))]
    workers = pool_workers()
    scale = w.head_dim ** -0.5
    rows, refs = [], []
    t_setup = time.perf_counter()
    with RowPool(k, v, iq, pq, ik, pk, workers) as pool:
        def round_(sel):
            bi = torch.tensor([r[0] for r in sel], device=q.device)
            ti = torch.tensor([r[1] for r in sel], device=q.device)
            qr = q[bi, ti].to("cpu", torch.float64).numpy()
            dr = do[bi, ti].to("cpu", torch.float64).numpy()
            return pool.dq(qr, dr, sel, scale=scale, causal=w.causal, window=w.window)

        round_(order[:workers])   # starts the workers; not timed
        setup_s = time.perf_counter() - t_setup
        i = workers
        t0 = time.perf_counter()
        while i < len(order) and time.perf_counter() - t0 < budget_s:
            sel = order[i:i + 2 * workers]
            i += len(sel)
            refs.append(round_(sel))
            rows += sel
        dt = time.perf_counter() - t0
    pairs = sum(int(oracle.visible(iq[b, t:t + 1], pq[b, t:t + 1], ik[b], pk[b], w.causal,
                                   w.window).sum()) for b, t in rows)
    flops = 2.0 * (2 * w.head_dim + w.dv) * w.num_q_heads * pairs
    base = {"value": flops / dt / 1e12 if dt > 0 else 0.0, "unit": "TFLOP/s", "kind": "oracle",
            **_host_info(workers),
            "sample": f"dQ of {len(rows)} random valid query rows of shard 0 x all "
                      f"{w.num_q_heads} heads ({pairs} visible pairs, {flops / 1e9:.1f} GFLOP fp64 "
                      f"at 2*(2D+Dv)*Hq per pair) in {dt:.1f} s over {workers} worker processes",
            "setup_s": setup_s}
    check = None
    if dq is not None and rows:
        ref = np.concatenate(refs)
        bi = torch.tensor([r[0] for r in rows], device=dq.device)
        ti = torch.tensor([r[1] for r in rows], device=dq.device)
        got = dq[bi, ti].to("cpu", torch.float64).numpy()
        err = got - ref
        check = {"rows": len(rows), "heads": w.num_q_heads,
                 "dq_rel_fro": float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)),
                 "dq_max_err_over_max_abs": float(np.abs(err).max() / max(np.abs(ref).max(), 1e-300))}
    return base, check


BWD_METRIC = "attention bwd TFLOP/s (visible pairs, 2*(3D+2Dv)*Hq per pair) + % of bf16 MFMA peak, 1 MI355X"


def bench_backward(args, w, dev):
    """attn_bwd over every shard of the all-gather strategy: shard r's queries
    (striped reorder) against the whole gathered K/V, with dout ~ N(0, 1).
    One step computes dq of every query and each shard's dk/dv contribution
    (what a reduce-scatter would sum across devices).  FLOPs count only visible
    pairs, 2 * (3 * D + 2 * Dv) * Hq per pair (the five products S, dK and dQ
    over Q/K's head dim D, dP and dV over V's head dim Dv; 10 * D * Hq when
    they are equal)."""
    if w.cp_size > 1:
        w = dataclasses.replace(w, reorder="striped", stripe=args.stripe)
    desc = w.describe()
    if w.cp_size > 1:
        desc = desc.replace(f"{w.cp_size} shards x {w.cp_size} ring steps",
                            f"{w.cp_size} shards (stripe {w.stripe}), each against the whole "
                            "gathered K/V in one call")
    log(f"backward, workload {w.cfg} {w.name}: {desc}")
    q, k, v, ids, pos = make_inputs(w, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 17)
    do = torch.randn(q.shape[:3] + (w.dv,), generator=g, device=dev).to(torch.bfloat16)
    cp = max(1, w.cp_size)
    if cp > 1:
        q, k, v, ids, pos, do = (bosf.reorder(t, cp, w.reorder, w.stripe) for t in (q, k, v, ids, pos, do))
    n = w.seq_len // cp
    gdt = torch.float32 if args.grad_dtype == "f32" else torch.bfloat16
    shards = []
    for r in range(cp):
        sl = slice(r * n, (r + 1) * n)
        qs, ds = q[:, sl].contiguous(), do[:, sl].contiguous()
        iq, pq = ids[:, sl], pos[:, sl]
        o, lse = bosf.attn_fwd(qs, k, v, iq, pq, ids, pos, causal=w.causal, window=w.window)
        dk = torch.empty(k.shape, dtype=gdt, device=dev)
        dv = torch.empty(v.shape, dtype=gdt, device=dev)
        dq = torch.empty(qs.shape, dtype=gdt, device=dev)
        shards.append((qs, ds, iq, pq, o, lse, dq, dk, dv))
    del q, do
    bdesc = bosf.make_desc(w.batch, n, w.seq_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           strides={"q_meta_batch_stride": ids.stride(0), "v_head_dim": w.dv})
    wsp = torch.empty(bosf.bwd_workspace_size(bdesc), dtype=torch.uint8, device=dev)
    log(f"backward workspace {wsp.numel() / 2**30:.2f} GiB")
    visible = visible_pairs(w, ids, pos, k.dtype)
    flops = 2.0 * (3 * w.head_dim + 2 * w.dv) * w.num_q_heads * visible
    log(f"visible pairs {visible}, {flops / 1e12:.3f} TFLOP per backward step")
    stream = torch.cuda.current_stream(dev)
    evs = []

    def step(record):
        for (qs, ds, iq, pq, o, lse, dq, dk, dv) in shards:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            bosf.attn_bwd(qs, k, v, iq, pq, ids, pos, o, lse, ds, causal=w.causal,
                          window=w.window, grad_dtype=gdt, dq=dq, dk=dk, dv=dv, workspace=wsp)
            if record:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record(stream)
                evs.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1000.0 / args.steps
    value = flops / (ms_step / 1000.0) / 1e12
    calls = [a.elapsed_time(b) for a, b in evs]
    call_ms = float(np.mean(calls))
    achieved = flops / cp / (call_ms / 1000.0) / 1e12
    log(f"{ms_step:.3f} ms/step, {value:.1f} TFLOP/s; attn_bwd {call_ms:.3f} ms per call")
    cpu = check = None
    if not args.no_cpu_baseline:
        log("timing the fp64 backward oracle on a host row sample")
        qs, ds, iq, pq = shards[0][:4]
        cpu, check = cpu_baseline_bwd(w, qs, k, v, ds, iq, pq, ids, pos, args.cpu_seconds,
                                      dq=shards[0][6])
    line = {
        "metric": BWD_METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "config": {"workload": f"{w.name} backward{' all-gather' if cp > 1 else ''}: {desc}",
                   "batch": w.batch, "seq_len": w.seq_len, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "v_head_dim": w.dv,
                   "window": list(w.window), "cp_shards": cp, "reorder": w.reorder,
                   "stripe": w.stripe, "grad_dtype": args.grad_dtype},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": "attn_bwd call (prep, both classifications, packing, dq and "
                               "dk/dv passes)",
                     "per_launch_flops": flops / cp},
        "cpu_baseline": cpu,
        "sample_parity": check,
        "detail": {"attn_bwd_calls_per_step": cp, "attn_bwd_avg_ms_per_call": call_ms,
                   "visible_pairs_per_step": visible,
                   "workspace_bytes": int(wsp.numel())},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
