"""GPU parity of the attention forward against the fp64 oracle.

Every case feeds the same seeded host (or torch-RNG device) tensors to the
HIP path through the C ABI and to the oracle, and holds the result to the bar
in ``_parity.compare``.  Small cases span several tiles with ragged tails,
all GQA group sizes (every workgroup shape of the bf16 kernel), both head
dims, both input dtypes, masked and unmasked, windows at their edges,
cross-attention with unrelated layouts, and empty inputs.
"""

import dataclasses

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare, to64
from _workload_io import (closed_form_counts, device_inputs, sample_rows, stratified_rows,
                          tiles_covered)
from workloads import get, packed_metadata, random_layout, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _dev(*ts):
    return [t.to(DEV) for t in ts]


# (B, Tq, Tk, Hq, Hkv, D, dtype, causal, window, self_attention)
SMALL = [
    (1, 1, 1, 1, 1, 64, "bf16", True, (-1, -1), True),
    (1, 33, 33, 8, 8, 128, "bf16", True, (-1, -1), True),
    (2, 257, 257, 16, 2, 128, "bf16", True, (-1, -1), True),
    (2, 300, 300, 16, 2, 128, "bf16", True, (40, 0), True),
    (1, 517, 517, 64, 8, 128, "bf16", True, (100, 0), True),
    (2, 200, 200, 32, 2, 128, "bf16", True, (0, 0), True),
    (2, 190, 190, 4, 1, 64, "bf16", False, (-1, -1), True),
    (1, 250, 250, 8, 4, 64, "bf16", False, (17, 9), True),
    (2, 129, 129, 3, 1, 128, "bf16", True, (-1, 5), True),
    (1, 300, 300, 12, 1, 128, "bf16", True, (-1, -1), True),
    (2, 161, 161, 6, 3, 64, "bf16", True, (30, 30), True),
    (1, 96, 96, 1, 1, 128, "bf16", True, (-1, -1), True),
    (2, 300, 517, 16, 2, 128, "bf16", True, (-1, -1), False),
    (1, 517, 300, 8, 2, 64, "bf16", False, (50, 50), False),
    (2, 64, 640, 16, 1, 128, "bf16", True, (200, 0), False),
    # 45 work items in runs of 6: counts rise along each run, so the runs are
    # dealt in reverse, the last one with 3 items and 3 positions past the end
    (1, 1440, 1440, 8, 1, 128, "bf16", True, (-1, -1), True),
    (1, 1440, 1440, 8, 1, 128, "bf16", True, (300, 0), True),
    (1, 256, 256, 4, 4, 64, "f32", True, (-1, -1), True),
    (2, 111, 111, 4, 2, 128, "f32", True, (20, 0), True),
    (1, 99, 140, 6, 1, 64, "f32", False, (-1, 3), False),
    (2, 70, 70, 2, 2, 128, "f32", True, (0, 0), True),
    # fp32 kernel: 45 items (9 heads x 5 query tiles of 64) in runs of 6, the
    # last one rising (dealt in reverse) with 3 positions past the end
    (1, 320, 320, 9, 3, 64, "f32", True, (-1, -1), True),
]


def _case_id(c):
    b, tq, tk, hq, hkv, d, dt, causal, w, self_ = c
    return f"B{b}_Tq{tq}_Tk{tk}_H{hq}-{hkv}_D{d}_{dt}_{'c' if causal else 'nc'}_w{w[0]}.{w[1]}_{'self' if self_ else 'cross'}"


@pytest.mark.parametrize("case", SMALL, ids=[_case_id(c) for c in SMALL])
@pytest.mark.parametrize("out", ["same", "f32"])
def test_small_random_layouts(case, out):
    b, tq, tk, hq, hkv, d, dt, causal, window, self_ = case
    rng = np.random.default_rng(tq * 7 + tk + hq)
    q_ids, q_pos = random_layout(rng, b, tq, max_segments=4, pad_prob=0.25, pos_offset_max=3)
    if self_:
        kv_ids, kv_pos = q_ids, q_pos
    else:
        kv_ids, kv_pos = random_layout(rng, b, tk, max_segments=3, pad_prob=0.25, pos_offset_max=40)
    q, k, v = random_qkv(b, tq, tk, hq, hkv, d, dt, seed=tq + tk)
    out_dtype = torch.float32 if out == "f32" else None
    o, lse = bosf.attn_fwd(*_dev(q, k, v, q_ids, q_pos, kv_ids, kv_pos), causal=causal,
                           window=window, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, q_ids, q_pos, kv_ids, kv_pos, causal=causal, window=window)
    compare(o, lse, ro, rl, dt, _case_id(case))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_negative_segment_ids(dt, causal):
    """Segment ids of either sign (0 still marks padding): padding queries see
    nothing, also next to keys whose id is -1, on boundary tiles as well as
    skipped and full ones."""
    rng = np.random.default_rng(71 if causal else 72)
    q_ids, q_pos = random_layout(rng, 2, 333, max_segments=6, pad_prob=0.4, pos_offset_max=3)
    sign = torch.from_numpy(np.where(rng.random(q_ids.shape) < 0.5, -1, 1).astype(np.int32))
    # every segment id negated (-1, -2, ...), then a few segments made positive again
    q_ids = torch.where(q_ids != 0, -q_ids, q_ids)
    q_ids = torch.where((q_ids < -3) & (sign > 0), -q_ids, q_ids)
    q, k, v = random_qkv(2, 333, 333, 16, 2, 128 if dt == "bf16" else 64, dt, seed=73)
    o, lse = bosf.attn_fwd(*_dev(q, k, v, q_ids, q_pos, q_ids, q_pos), causal=causal,
                           window=(70, 0) if causal else (60, 60))
    ro, rl = oracle.attention(q, k, v, q_ids, q_pos, q_ids, q_pos, causal=causal,
                              window=(70, 0) if causal else (60, 60))
    assert (q_ids == -1).any() and (q_ids == 0).any()
    compare(o, lse, ro, rl, dt, f"negative ids {dt} causal={causal}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prepared_forward_reuses_schedule_and_packing(dt):
    """The forward with its workspace in two parts (ra_attn_fwd_ex): bit-identical
    to ra_attn_fwd when it writes both parts, and when it reuses the schedule
    and/or the packed K/V written by an earlier call on the same layout and
    K/V -- also for another query range against the same K/V (packing reused,
    schedule rewritten) and for the accumulating forward."""
    rng = np.random.default_rng(81)
    ids, pos = random_layout(rng, 2, 400, max_segments=4, pad_prob=0.2, pos_offset_max=3)
    d = 128 if dt == "bf16" else 64
    q, k, v = _dev(*random_qkv(2, 400, 400, 16, 2, d, dt, seed=82))
    ids, pos = _dev(ids, pos)
    kw = dict(causal=True, window=(90, 0))
    ref = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, **kw)
    desc = bosf.make_desc(2, 400, 400, 16, 2, d, 0 if dt == "bf16" else 1, window=(90, 0))
    sb, kb = bosf.workspace_parts(desc)
    sched = torch.empty(sb, dtype=torch.uint8, device=DEV)
    kvw = torch.empty(max(kb, 1), dtype=torch.uint8, device=DEV)
    both = bosf.FWD_SCHEDULE_READY | bosf.FWD_KV_READY
    for flags in (0, both, bosf.FWD_SCHEDULE_READY, bosf.FWD_KV_READY, both):
        got = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, prepared=(sched, kvw, flags), **kw)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), flags
    # the second half of the queries against the same K/V: the packing is reused
    sub = slice(200, 400)
    ref2 = bosf.attn_fwd(q[:, sub], k, v, ids[:, sub], pos[:, sub], ids, pos, **kw)
    got2 = bosf.attn_fwd(q[:, sub], k, v, ids[:, sub], pos[:, sub], ids, pos,
                         prepared=(sched, kvw, bosf.FWD_KV_READY), **kw)
    assert torch.equal(got2[0], ref2[0]) and torch.equal(got2[1], ref2[1])
    # accumulating forward on a partial, in place, with both parts reused
    g = torch.Generator().manual_seed(83)
    po = torch.randn((2, 400, 16, d), generator=g).to(DEV)
    pl = torch.randn((2, 400, 16), generator=g).to(DEV)
    ra_ = bosf.attn_fwd_accumulate(q, k, v, ids, pos, ids, pos, po.clone(), pl.clone(), **kw)
    bosf.attn_fwd(q, k, v, ids, pos, ids, pos, prepared=(sched, kvw, 0), **kw)
    ga = bosf.attn_fwd_accumulate(q, k, v, ids, pos, ids, pos, po.clone(), pl.clone(),
                                  prepared=(sched, kvw, both), **kw)
    assert torch.equal(ga[0], ra_[0]) and torch.equal(ga[1], ra_[1])
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), ids.cpu(), pos.cpu(), ids.cpu(),
                              pos.cpu(), **kw)
    compare(got[0], got[1], ro, rl, dt, "prepared forward")


def test_packed_layout_scale_and_window_edges():
    """Packed slots with padding; a non-default scale; window exactly at 31/32/33."""
    ids, pos = packed_metadata(2, 512, 2, 200)
    q, k, v = random_qkv(2, 512, 512, 16, 2, 128, "bf16", seed=3)
    for window in [(31, 0), (32, 0), (33, 0)]:
        o, lse = bosf.attn_fwd(*_dev(q, k, v, ids, pos, ids, pos), scale=0.05, window=window)
        ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, scale=0.05, window=window)
        compare(o, lse, ro, rl, "bf16", f"window {window}")


def test_empty_inputs():
    q, k, v = random_qkv(2, 40, 0, 8, 2, 128, "bf16", seed=1)
    ids = torch.ones(2, 40, dtype=torch.int32)
    pos = torch.arange(40, dtype=torch.int32).repeat(2, 1)
    kid = torch.ones(2, 0, dtype=torch.int32)
    o, lse = bosf.attn_fwd(*_dev(q, k, v, ids, pos, kid, kid))
    assert (o == 0).all() and torch.isneginf(lse).all()
    # no queries / no batch: nothing to do, must not fail
    q0 = torch.zeros(2, 0, 8, 128, dtype=torch.bfloat16)
    e = torch.zeros(2, 0, dtype=torch.int32)
    k1, v1 = random_qkv(2, 8, 8, 8, 2, 128, "bf16")[1:]
    i1 = torch.ones(2, 8, dtype=torch.int32)
    o0, l0 = bosf.attn_fwd(*_dev(q0, k1, v1, e, e, i1, i1))
    assert o0.shape == (2, 0, 8, 128)
    qb = torch.zeros(0, 5, 8, 128, dtype=torch.bfloat16)
    eb = torch.zeros(0, 5, dtype=torch.int32)
    kb = torch.zeros(0, 5, 2, 128, dtype=torch.bfloat16)
    ob, lb = bosf.attn_fwd(*_dev(qb, kb, kb, eb, eb, eb, eb))
    assert ob.numel() == 0


def test_all_padding_queries():
    ids = torch.zeros(1, 100, dtype=torch.int32)
    pos = torch.arange(100, dtype=torch.int32)[None]
    q, k, v = random_qkv(1, 100, 100, 8, 1, 128, "bf16", seed=2)
    o, lse = bosf.attn_fwd(*_dev(q, k, v, ids, pos, ids, pos))
    assert (o == 0).all() and torch.isneginf(lse).all()


def test_batch_strided_views():
    """Q/K/V/O/LSE and metadata as views into longer sequences (ring shards)."""
    ids, pos = packed_metadata(2, 1024, 2, 400)
    q, k, v = random_qkv(2, 1024, 1024, 16, 2, 128, "bf16", seed=5)
    qd, kd, vd, idd, posd = _dev(q, k, v, ids, pos)
    o_full = torch.full((2, 1024, 16, 128), 7.0, dtype=torch.float32, device=DEV)
    l_full = torch.full((2, 1024, 16), 7.0, dtype=torch.float32, device=DEV)
    qs, ks = slice(256, 512), slice(512, 1024)
    o, lse = bosf.attn_fwd(qd[:, qs], kd[:, ks], vd[:, ks], idd[:, qs], posd[:, qs], idd[:, ks],
                           posd[:, ks], causal=False, window=(300, 300), out_dtype=torch.float32,
                           out=o_full[:, qs], lse=l_full[:, qs])
    ro, rl = oracle.attention(q[:, qs], k[:, ks], v[:, ks], ids[:, qs], pos[:, qs], ids[:, ks],
                              pos[:, ks], causal=False, window=(300, 300))
    compare(o_full[:, qs], l_full[:, qs], ro, rl, "bf16", "views")
    # untouched outside the view
    assert (o_full[:, :256] == 7).all() and (o_full[:, 512:] == 7).all()
    assert (l_full[:, :256] == 7).all() and (l_full[:, 512:] == 7).all()


def test_deterministic():
    ids, pos = packed_metadata(2, 2048, 2, 900)
    q, k, v = _dev(*random_qkv(2, 2048, 2048, 16, 2, 128, "bf16", seed=9))
    idd, posd = _dev(ids, pos)
    o1, l1 = bosf.attn_fwd(q, k, v, idd, posd, idd, posd, window=(500, 0))
    o2, l2 = bosf.attn_fwd(q, k, v, idd, posd, idd, posd, window=(500, 0))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# --------------------------------------------------------------------------- workloads 1 and 2

@pytest.mark.parametrize("cfg", [1, 2])
def test_workload_full(cfg):
    w = get(cfg)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    q, k, v = random_qkv(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                         w.head_dim, w.dtype, seed=w.seed)
    o, lse = bosf.attn_fwd(*_dev(q, k, v, ids, pos, ids, pos), causal=w.causal, window=w.window)
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window)
    e = compare(o, lse, ro, rl, w.dtype, w.name)
    print(f"{w.name}: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")


@pytest.mark.parametrize("fused", [True, False])
def test_workload3_ring_emulation(fused):
    """Workload 3: dual-chunk reorder, 4 shards x 4 ring steps (merged in the
    forward's epilogue, or by attn_merge), inverse reorder -- against one
    unsplit oracle attention."""
    w = get(3)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    q, k, v = random_qkv(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                         w.head_dim, w.dtype, seed=w.seed)
    o, lse = bosf.ring_forward(*_dev(q, k, v, ids, pos), w.cp_size, w.reorder, w.stripe,
                               causal=w.causal, window=w.window, fused=fused)
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window)
    e = compare(o, lse, ro, rl, "bf16", w.name)
    print(f"{w.name} fused={fused}: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")


@pytest.mark.parametrize("kind,stripe,window,partial,fused", [
    ("striped", 1, (-1, -1), torch.float32, True), ("striped", 1, (-1, -1), torch.float32, False),
    ("dual_chunk", 1, (700, 0), torch.bfloat16, True),
    ("dual_chunk", 1, (700, 0), torch.bfloat16, False),
    ("striped", 64, (300, 0), torch.float32, True)])
def test_ring_variants(kind, stripe, window, partial, fused):
    ids, pos = packed_metadata(2, 2048, 4, 400)
    q, k, v = random_qkv(2, 2048, 2048, 16, 2, 128, "bf16", seed=12)
    o, lse = bosf.ring_forward(*_dev(q, k, v, ids, pos), 4, kind, stripe, window=window,
                               partial_dtype=partial, fused=fused)
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, window=window)
    compare(o, lse, ro, rl, "bf16", f"ring {kind} {stripe} fused={fused}")


def _random_partial(b, t, h, d, dtype, seed, empty_frac=0.25):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn((b, t, h, d), generator=g).to(dtype)
    lse = torch.randn((b, t, h), generator=g) * 3
    empty = torch.rand((b, t, h), generator=g) < empty_frac
    lse[empty] = -np.inf
    o[empty] = 0
    return o, lse


@pytest.mark.parametrize("qkv_dt,part_dt,out_dt,in_place", [
    ("bf16", torch.float32, torch.float32, True), ("bf16", torch.float32, torch.bfloat16, False),
    ("bf16", torch.bfloat16, torch.bfloat16, True), ("bf16", torch.bfloat16, torch.float32, False),
    ("f32", torch.float32, torch.float32, True), ("f32", torch.float32, torch.bfloat16, False)])
def test_accumulate_equals_merge_of_attention_and_partial(qkv_dt, part_dt, out_dt, in_place):
    """attn_fwd_accumulate = merge(attention over this call's keys, partial)."""
    rng = np.random.default_rng(7)
    b, tq, tk, hq, hkv, d = 2, 300, 260, 8, 2, 128
    q_ids, q_pos = random_layout(rng, b, tq, max_segments=3, pad_prob=0.2)
    k_ids, k_pos = random_layout(rng, b, tk, max_segments=3, pad_prob=0.2, pos_offset_max=50)
    q, k, v = random_qkv(b, tq, tk, hq, hkv, d, qkv_dt, seed=8)
    po, pl = _random_partial(b, tq, hq, d, part_dt, 9)
    po_d, pl_d = po.to(DEV), pl.to(DEV)
    kw = dict(window=(40, 0))
    if in_place:
        o, lse = bosf.attn_fwd_accumulate(*_dev(q, k, v, q_ids, q_pos, k_ids, k_pos), po_d, pl_d,
                                          **kw)
        assert o.data_ptr() == po_d.data_ptr()
    else:
        out = torch.empty((b, tq, hq, d), dtype=out_dt, device=DEV)
        lout = torch.empty((b, tq, hq), device=DEV)
        o, lse = bosf.attn_fwd_accumulate(*_dev(q, k, v, q_ids, q_pos, k_ids, k_pos), po_d, pl_d,
                                          out=out, lse=lout, **kw)
    ao, al = oracle.attention(q, k, v, q_ids, q_pos, k_ids, k_pos, **kw)
    ro, rl = oracle.merge(ao, al, po, pl)
    compare(o, lse, ro, rl, "bf16", f"accumulate {qkv_dt} {part_dt}->{out_dt} in_place={in_place}")


def test_accumulate_in_place_leaves_untouched_tiles_bit_exact():
    """Query tiles with nothing visible in this call keep their partial bits."""
    ids, pos = packed_metadata(1, 512, 1, 512)
    q, k, v = random_qkv(1, 512, 512, 8, 1, 128, "bf16", seed=4)
    po, pl = _random_partial(1, 512, 8, 128, torch.float32, 5, empty_frac=0.0)
    po_d, pl_d = po.to(DEV), pl.to(DEV)
    # keys are the last 64 positions: query tokens 0..447 see nothing (causal)
    bosf.attn_fwd_accumulate(*_dev(q, k[:, 448:], v[:, 448:], ids, pos, ids[:, 448:],
                                   pos[:, 448:]), po_d, pl_d)
    assert torch.equal(po_d[:, :448].cpu(), po[:, :448])
    assert torch.equal(pl_d[:, :448].cpu(), pl[:, :448])
    ao, al = oracle.attention(q, k[:, 448:], v[:, 448:], ids, pos, ids[:, 448:], pos[:, 448:])
    ro, rl = oracle.merge(ao, al, po, pl)
    compare(po_d, pl_d, ro, rl, "bf16", "accumulate tail")


# --------------------------------------------------------------------------- workloads 4 and 5

def _run_workload(w, q, k, v, ids, pos):
    if w.cp_size > 1:
        # the benchmark's schedule: per-stripe plan (Q read in place when every
        # call covers one stripe), inverse reorder folded into the stores
        plan = bosf.ring_plan(ids, pos, w.cp_size, w.reorder, w.stripe,
                              num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                              head_dim=w.head_dim, dtype=q.dtype, causal=w.causal,
                              window=w.window, halves=w.reorder == "dual_chunk")
        return bosf.ring_forward(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe,
                                 causal=w.causal, window=w.window, plan=plan)
    return bosf.attn_fwd(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window)


@pytest.fixture(scope="module")
def full_size_oracle():
    """Per workload (4 or 5): the full-size inputs on the device, a row sample
    holding one row of every 32-token query tile of every launch (unsplit,
    dual-chunk and striped(1) rings alike) plus segment starts, window edges,
    padding and shard boundaries, and the oracle's O and LSE on those rows,
    every head.  One workload is held at a time."""
    cache = {}

    def case(cfg):
        if cfg not in cache:
            cache.clear()
            w = get(cfg)
            inputs = device_inputs(w)
            rng = np.random.default_rng(cfg)
            left = w.window[0]
            edges = [0, 1, 2, 31, 32, 63, 64, left - 1, left, left + 1, left + 2,
                     w.valid_per_slot - 1, w.valid_per_slot, w.slot_len - 1]
            rows = set(stratified_rows(w, rng)) | set(sample_rows(w, rng, edges, n_random=0))
            n = w.seq_len // 4
            for kind in ("dual_chunk", "striped"):   # both sides of every shard boundary
                m = oracle.reorder_map(w.seq_len, 4, kind, 1)
                for r in range(1, 4):
                    for p in (r * n - 1, r * n, r * n + n // 2 - 1, r * n + n // 2):
                        rows.add((0, int(m[p])))
            rows = sorted(rows)
            q, k, v, ids, pos = inputs
            ro, rl = oracle.attention_rows(q, k, v, ids, pos, ids, pos, rows, causal=w.causal,
                                           window=w.window)
            cache[cfg] = (w, inputs, rows, ro, rl)
        return cache[cfg]

    yield case
    cache.clear()


@pytest.mark.parametrize("cfg,kind", [(4, None), (5, "dual_chunk"), (5, "striped")])
def test_workload_full_size_stratified(full_size_oracle, cfg, kind):
    """Full-size run in the benchmark's configuration (workload 5 also under
    the tutorial's ring layout, striped with stripe 1), compared with the
    oracle on at least one row of every 32-token query tile of every launch,
    every head."""
    w, inputs, rows, ro, rl = full_size_oracle(cfg)
    if kind is not None:
        w = dataclasses.replace(w, reorder=kind, stripe=1)
        order = oracle.reorder_map(w.seq_len, w.cp_size, kind, 1)
    else:
        order = np.arange(w.seq_len)
    bm = bosf.tile_shape(bosf.make_desc(1, 1, 1, w.num_q_heads, w.num_kv_heads, w.head_dim))[0]
    assert bm == 32
    assert len(tiles_covered(rows, order, bm)) == w.batch * w.seq_len // bm
    o, lse = _run_workload(w, *inputs)
    torch.cuda.synchronize()
    bi = torch.tensor([r[0] for r in rows])
    ti = torch.tensor([r[1] for r in rows])
    e = compare(o[bi, ti], lse[bi, ti], ro, rl, "bf16", f"{w.name} {kind}")
    print(f"{w.name} {kind or ''}: {len(rows)} rows x {w.num_q_heads} heads: max|dO|={e[0]:.2e} "
          f"max|dLSE|={e[1]:.2e}")


@pytest.mark.parametrize("cfg,kind", [(2, None), (4, None), (5, None), (5, "striped")])
def test_workload_zero_queries_every_row(cfg, kind):
    """Q = 0: every row's LSE is ln(visible keys), known in closed form for
    every row at full size; padding rows are -inf."""
    w = get(cfg)
    if kind is not None:
        w = dataclasses.replace(w, reorder=kind, stripe=1)
    q, k, v, ids, pos = device_inputs(w, zero_q=True)
    o, lse = _run_workload(w, q, k, v, ids, pos)
    n = closed_form_counts(w, pos, ids)                 # [B, T]
    ref = torch.where(n > 0, torch.log(n), torch.full_like(n, -np.inf))
    got = lse.to(torch.float64)
    live = n > 0
    assert torch.equal(torch.isneginf(got), ~live[:, :, None].expand_as(got))
    err = (got - ref[:, :, None])[live[:, :, None].expand_as(got)].abs().max().item()
    assert err <= 1e-5, err
    assert (o[~live] == 0).all()


@pytest.mark.parametrize("cfg,kind", [(4, None), (5, None), (5, "striped")])
def test_workload_uniform_v_every_row(cfg, kind):
    """v[b, j, g, :] = c_g: every live row's output is c_g of its head's group."""
    w = get(cfg)
    if kind is not None:
        w = dataclasses.replace(w, reorder=kind, stripe=1)
    c = torch.randn((w.num_kv_heads, w.head_dim), generator=torch.Generator().manual_seed(1))
    c = c.to(torch.bfloat16)
    q, k, v, ids, pos = device_inputs(w, uniform_v=c)
    o, lse = _run_workload(w, q, k, v, ids, pos)
    ref = c.to(DEV, torch.float32).repeat_interleave(w.group, dim=0)   # [Hq, D]
    live = ids != 0
    err = (o[live].float() - ref[None]).abs().max().item()
    assert err <= 2e-2, err
    assert torch.isneginf(lse[~live]).all() and (o[~live] == 0).all()


def _ramp_inputs(kind, b=1, tq=256, tk=1024, hq=8, hkv=1, d=128):
    """Q and K whose scores sweep a range of ~300 natural-log units: rising
    along the keys (the running max must be raised on every tile), falling
    (the first tile holds the max and later probabilities underflow to 0), or
    random with a spread of ~+-100."""
    g = torch.Generator().manual_seed({"up": 11, "down": 12, "wide": 13}[kind])
    v = torch.randn((b, tk, hkv, d), generator=g).to(torch.bfloat16)
    if kind == "wide":
        q = (6.0 * torch.randn((b, tq, hq, d), generator=g)).to(torch.bfloat16)
        k = (6.0 * torch.randn((b, tk, hkv, d), generator=g)).to(torch.bfloat16)
        return q, k, v
    q = torch.ones((b, tq, hq, d)).to(torch.bfloat16)
    j = torch.arange(tk, dtype=torch.float32)
    ramp = (j if kind == "up" else tk - 1 - j) / tk * 26.5
    k = ramp[None, :, None, None].expand(b, tk, hkv, d).to(torch.bfloat16).contiguous()
    return q, k, v


@pytest.mark.parametrize("kind", ["up", "down", "wide"])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_over_wide_score_ranges(kind, causal):
    """The lazy running max: raised on (nearly) every tile, never raised, and
    raised at random, with O and LSE against the oracle.  Without the rescale
    the rising case would overflow (e^300)."""
    q, k, v = _ramp_inputs(kind)
    tq, tk = q.shape[1], k.shape[1]
    qi = torch.ones((1, tq), dtype=torch.int32)
    ki = torch.ones((1, tk), dtype=torch.int32)
    qp = torch.arange(tk - tq, tk, dtype=torch.int32)[None]   # queries see every key causally
    kp = torch.arange(tk, dtype=torch.int32)[None]
    o, lse = bosf.attn_fwd(*_dev(q, k, v, qi, qp, ki, kp), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, qi, qp, ki, kp, causal=causal)
    e = compare(o, lse, ro, rl, "bf16", f"{kind} causal={causal}")
    print(f"{kind} causal={causal}: LSE range {rl.min():.1f}..{rl.max():.1f}, "
          f"max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")
