"""Benchmark: attention forward TFLOP/s on visible (query, key) pairs, one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  For the default workload (one device's share of the
TransformerEngine tutorial's long-context case, run as a 4-shard ring) that is:
causal load-balancing reorder of Q, K, V, segment ids and positions; for each
of the 4 shards, 4 ring steps -- attn_fwd for the shard's own chunk, then
attn_fwd_accumulate for the 3 chunks that arrive next, each folding its block
into the running fp32 partial in its epilogue (the merge of the ring update,
fused; ``--unfused`` runs attn_fwd + attn_merge instead); inverse reorder of O
and LSE, folded into the forward's stores (a dual-chunk shard is two
contiguous stripes of the sequence, written with a split output at their
original positions).  A plan computed once per layout skips the ring steps
whose blocks hold no visible pair and finishes each stripe at its own last
step with work (``--plan-by-rank``, ``--no-plan`` for the coarser schedules).
All four shards are computed, so a step
is the complete forward of B=2 x 65536 tokens; FLOPs count only visible pairs
(4 * head_dim * Hq per pair).  attn_merge and the inverse reorder kernel are
also timed on their own at the step's shapes.

Prints one JSON line.  ``roofline`` is measured live with HIP events that the
library records on its stream right before and after the attention kernel of
every forward call (``ra_profile_next_kernel``; the call's tile classification
and K/V repack fall outside); ``cpu_baseline`` times the fp64 oracle on a
bounded row sample of the same inputs.
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


def cpu_baseline(w, q, k, v, ids, pos, budget_s, o=None, lse=None):
    """Oracle (fp64, host) on a bounded random row sample of the same inputs.

    With the step's output (``o``, ``lse`` in token order), the oracle rows it
    computes are also compared with the GPU's: returns the baseline and the
    sample's max |O| and |LSE| differences and -inf mismatch count (or None)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    kc, vc, idc, posc = k.cpu(), v.cpu(), ids.cpu(), pos.cpu()
    rng = np.random.default_rng(0)
    valid = np.argwhere(idc.numpy() != 0)
    order = rng.permutation(len(valid))
    rows, refs, pairs, t0 = [], [], 0, time.perf_counter()
    for j in order:
        b, i = int(valid[j][0]), int(valid[j][1])
        refs.append(oracle.attention_rows(q, kc, vc, idc, posc, idc, posc, [(b, i)],
                                          causal=w.causal, window=w.window))
        n = int(oracle.visible(idc[b, i:i + 1], posc[b, i:i + 1], idc[b], posc[b], w.causal,
                               w.window).sum())
        rows.append((b, i))
        pairs += n
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 2.0 * (w.head_dim + w.dv) * w.num_q_heads * pairs
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} random valid query rows x all {w.num_q_heads} heads "
                      f"({pairs} visible pairs, {flops / 1e9:.1f} GFLOP fp64) in {dt:.1f} s"}
    check = None
    if o is not None and rows:
        o_err = l_err = 0.0
        mism = 0
        for (b, i), (ro, rl) in zip(rows, refs):
            go = o[b, i].to("cpu", torch.float64).numpy()
            gl = lse[b, i].to("cpu", torch.float64).numpy()
            ei, er = np.isneginf(gl), np.isneginf(rl[0])
            mism += int((ei != er).sum())
            live = ~(ei | er)
            o_err = max(o_err, float(np.abs(go - ro[0]).max()))
            if live.any():
                l_err = max(l_err, float(np.abs(gl[live] - rl[0][live]).max()))
        check = {"rows": len(rows), "heads": w.num_q_heads, "max_abs_o": o_err,
                 "max_abs_lse": l_err, "lse_neg_inf_mismatches": mism}
    return base, check


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=5, help="workload number (1-5)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    bosf.load_library()
    if args.backward:
        return bench_backward(args, w, dev)
    desc = w.describe()
    if allgather:
        desc = desc.replace(f"{w.cp_size} shards x {w.cp_size} ring steps",
                            f"{w.cp_size} shards (stripe {w.stripe}), each against the whole "
                            "gathered K/V in one call")
    log(f"workload {w.cfg} {w.name}: {desc}")
    q, k, v, ids, pos = make_inputs(w, dev)

    # Work of one step: visible pairs of the unsplit problem, counted by the
    # library's own classification pass (the ring decomposition covers every
    # visible pair exactly once).
    _, pairs = bosf.classify_tiles(ids, pos, ids, pos, num_q_heads=w.num_q_heads,
                                   num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                   v_head_dim=w.dv, dtype=q.dtype, causal=w.causal,
                                   window=w.window)
    visible = int(pairs.sum().item())
    # 2*D flops for Q K^T and 2*Dv for P V per visible pair and query head
    flops = 2.0 * (w.head_dim + w.dv) * w.num_q_heads * visible
    log(f"visible pairs {visible}, {flops / 1e12:.3f} TFLOP per step")

    ev = EventLog()
    out = {}
    if allgather:
        bufs = bosf.RingBuffers.like(q, k, ids, w.cp_size, partials=False)

        def step():
            out.clear()   # the previous step's output is not held across the next
            out["o"], out["lse"] = bosf.allgather_forward(
                q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, causal=w.causal,
                window=w.window, bufs=bufs, step_hook=ev.hook)
    elif w.cp_size > 1:
        bufs = bosf.RingBuffers.like(q, k, ids, w.cp_size)
        # The ring schedule of this segment layout (visible pairs per rank,
        # dual-chunk stripe and step), computed once outside the timed region
        # like the layout itself; steps whose blocks hold no visible pair are
        # then not launched, and each stripe is finished at its own last step
        # with work.
        plan = None
        if not args.no_plan and not args.unfused:
            plan = bosf.ring_plan(ids, pos, w.cp_size, w.reorder, w.stripe,
                                  num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                                  head_dim=w.head_dim, dtype=q.dtype, causal=w.causal,
                                  window=w.window,
                                  halves=w.reorder == "dual_chunk" and not args.plan_by_rank)
            log(f"ring plan (visible pairs per rank x step): {plan.tolist()}")

        def step():
            out.clear()   # the previous step's output is not held across the next
            out["o"], out["lse"] = bosf.ring_forward(
                q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, causal=w.causal,
                window=w.window, bufs=bufs, step_hook=ev.hook, fused=not args.unfused, plan=plan,
                fuse_inverse=not args.separate_inverse)
    else:
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

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev.enabled = True
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev.enabled = False
    ms_step = (t1 - t0) * 1000.0 / args.steps
    value = flops / (ms_step / 1000.0) / 1e12
    log(f"{ms_step:.3f} ms/step, {value:.1f} TFLOP/s")

    attn_ms = ev.ms("attn_fwd")          # whole library calls
    kern_ms = ev.ms("attn_kernel")       # the attention kernel of each call
    n_attn = len(attn_ms)
    attn_total_ms = float(sum(attn_ms))
    kern_total_ms = float(sum(kern_ms))
    per_launch_flops = flops * args.steps / n_attn
    achieved = flops * args.steps / (kern_total_ms / 1000.0) / 1e12
    per_step = n_attn // args.steps
    step_kern = [sum(kern_ms[i * per_step:(i + 1) * per_step]) for i in range(args.steps)]
    detail = {"attn_fwd_launches_per_step": per_step,
              "attn_kernel_ms_per_step": kern_total_ms / args.steps,
              "attn_kernel_ms_per_step_median": float(np.median(step_kern)),
              "attn_kernel_ms_per_step_min": float(min(step_kern)),
              "attn_kernel_avg_ms_per_launch": kern_total_ms / n_attn,
              "attn_fwd_call_ms_per_step": attn_total_ms / args.steps,
              "attn_fwd_call_avg_ms_per_launch": attn_total_ms / n_attn,
              "call_TFLOPs_incl_classify_pack": flops * args.steps / (attn_total_ms / 1000.0) / 1e12,
              "visible_pairs_per_step": visible,
              "pct_of_bf16_peak_whole_step": 100.0 * value / PEAK_BF16_TFLOPS}
    if w.cp_size > 1:
        # per rank: the attention kernel time of its share per step and, with
        # the ring plan's pair counts, its own rate (the headline aggregates
        # all ranks' flops over their summed kernel time)
        rk = ev.ranks("attn_kernel")
        rank_ms = [sum(m for m, r in zip(kern_ms, rk) if r == rr) / args.steps
                   for rr in range(w.cp_size)]
        detail["attn_kernel_ms_per_step_by_rank"] = rank_ms
        if not allgather and plan is not None:
            rank_tf = [2.0 * (w.head_dim + w.dv) * w.num_q_heads * float(plan[rr].sum())
                       / (rank_ms[rr] / 1000.0) / 1e12 for rr in range(w.cp_size)]
            detail["attn_kernel_TFLOPs_by_rank"] = rank_tf
            detail["attn_kernel_TFLOPs_min_rank"] = min(rank_tf)
        b, t, hq, d = q.shape
        n = t // w.cp_size
        reorder_ms = sum(ev.ms("reorder")) / args.steps
        inv_ms = sum(ev.ms("inverse_reorder")) / args.steps
        # Q is read in place (no reordered copy) when the per-stripe plan never
        # runs both stripes of a shard in one call
        q_moved = (allgather or args.unfused or args.separate_inverse or plan is None
                   or bosf.needs_reordered_q(plan, w.cp_size))
        fwd_bytes = 2 * ((q.numel() * 2 if q_moved else 0) + 2 * k.numel() * 2
                         + 2 * ids.numel() * 4)
        detail["q_reordered"] = bool(q_moved)
        inv_bytes = 2 * (q.numel() * 2 + b * t * hq * 4)
        detail.update({
            "strategy": ("all-gather: each shard against the whole K/V, no merge" if allgather
                         else "ring: unfused, attn_merge per step" if args.unfused
                         else "ring: merges fused into attn_fwd_accumulate epilogues, "
                              + ("every step launched" if args.no_plan
                                 else "steps without visible pairs skipped")),
            "reorder_ms_per_step": reorder_ms,
            "reorder_GBs": fwd_bytes / (reorder_ms / 1000.0) / 1e9,
        })
        if ev.ms("inverse_reorder"):
            detail.update({"inverse_reorder_ms_per_step": inv_ms,
                           "inverse_reorder_GBs": inv_bytes / (inv_ms / 1000.0) / 1e9})
        else:
            detail["inverse_reorder"] = ("folded into the forward's stores: each dual-chunk "
                                         "stripe's O and LSE are written at their original "
                                         "positions (split output)")
            # the inverse reorder kernel on its own, on the step's O and LSE
            # (outside the step), for its HBM rate
            o_s, l_s = out["o"], out["lse"]
            for _ in range(2):
                bosf.inverse_reorder(o_s, w.cp_size, w.reorder, w.stripe)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                bosf.inverse_reorder(o_s, w.cp_size, w.reorder, w.stripe)
                bosf.inverse_reorder(l_s, w.cp_size, w.reorder, w.stripe)
            e1.record()
            torch.cuda.synchronize()
            ims = e0.elapsed_time(e1) / 5
            detail.update({"inverse_reorder_standalone_ms": ims,
                           "inverse_reorder_standalone_GBs": inv_bytes / (ims / 1000.0) / 1e9})
        if args.unfused:
            merges = ev.ms("attn_merge")
            detail["attn_merge_ms_per_step"] = sum(merges) / args.steps
        # attn_merge on its own: two fp32 shard partials with finite LSE (every
        # row reads both operands): 3 * D * 4 + 12 bytes per (b, t, h) row.
        pa = torch.randn((b, n, hq, d), device=dev)
        pb = torch.randn_like(pa)
        la = torch.randn((b, n, hq), device=dev)
        lb = torch.randn_like(la)
        outm = torch.empty_like(pa)
        outl = torch.empty_like(la)
        for _ in range(2):
            bosf.attn_merge(pa, la, pb, lb, out=outm, lse_out=outl)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            bosf.attn_merge(pa, la, pb, lb, out=outm, lse_out=outl)
        e1.record()
        torch.cuda.synchronize()
        mms = e0.elapsed_time(e1) / 5
        mbytes = b * n * hq * (3 * 4 * d + 12)
        detail.update({"attn_merge_ms_per_call": mms,
                       "attn_merge_GBs": mbytes / (mms / 1000.0) / 1e9,
                       "attn_merge_bytes_per_call": mbytes})
        del pa, pb, la, lb, outm, outl
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": (measured_traffic(per_step) if args.workload == 5 and not allgather
                            and not args.unfused and not args.no_plan else None),
                "kernel": "attn_fwd_bf16_kernel (events recorded by the library around the "
                          "kernel alone)",
                "per_launch_flops": per_launch_flops}

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
    query rows: dQ of each row over all heads (products S, dP, dQ: 2*(2D+Dv)*Hq
    flops per visible pair, 6*D*Hq when D = Dv).  With the shard's dQ from the
    GPU, the sampled rows are also compared: relative Frobenius error and max
    error over max |dQ| of the sample (or None)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    qc, kc, vc, dc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    iq, pq, ik, pk = q_ids.cpu(), q_pos.cpu(), kv_ids.cpu(), kv_pos.cpu()
    rng = np.random.default_rng(1)
    valid = np.argwhere(iq.numpy() != 0)
    order = rng.permutation(len(valid))
    rows, refs, pairs, t0 = [], [], 0, time.perf_counter()
    for j in order:
        b, i = int(valid[j][0]), int(valid[j][1])
        refs.append(oracle.backward_query_rows(qc, kc, vc, dc, iq, pq, ik, pk, [(b, i)],
                                               causal=w.causal, window=w.window)[0])
        pairs += int(oracle.visible(iq[b, i:i + 1], pq[b, i:i + 1], ik[b], pk[b], w.causal,
                                    w.window).sum())
        rows.append((b, i))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 2.0 * (2 * w.head_dim + w.dv) * w.num_q_heads * pairs
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"dQ of {len(rows)} random valid query rows of shard 0 x all "
                      f"{w.num_q_heads} heads ({pairs} visible pairs, {flops / 1e9:.1f} GFLOP fp64 "
                      f"at 2*(2D+Dv)*Hq per pair) in {dt:.1f} s"}
    check = None
    if dq is not None and rows:
        ref = np.stack(refs)
        got = np.stack([dq[b, i].to("cpu", torch.float64).numpy() for b, i in rows])
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
    _, pairs = bosf.classify_tiles(ids, pos, ids, pos, num_q_heads=w.num_q_heads,
                                   num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                   v_head_dim=w.dv, dtype=k.dtype, causal=w.causal,
                                   window=w.window)
    visible = int(pairs.sum().item())
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
