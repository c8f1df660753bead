"""GPU parity of the all-gather context-parallel forward and of the ring plan.

Each rank's query shard of the striped reorder attends to the whole
(reordered) K/V in one call; the result, permuted back, must equal plain
attention over the original order.  Small cases cover several stripe sizes
and windows; the full-size case is the long-context workload's shape with the
tutorial's all-gather stripe size of 512, checked on sampled rows and, via
Q = 0, on every row.
"""

import dataclasses

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare
from _workload_io import closed_form_counts, device_inputs, sample_rows
from workloads import get, packed_metadata, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _dev(*ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("stripe,window,cp", [(1, (-1, -1), 4), (64, (256, 0), 4), (512, (-1, -1), 2),
                                              (32, (300, 0), 8)])
def test_allgather_small(stripe, window, cp):
    ids, pos = packed_metadata(2, 4096, 4, 700)
    q, k, v = random_qkv(2, 4096, 4096, 16, 2, 128, "bf16", seed=21)
    o, lse = bosf.allgather_forward(*_dev(q, k, v, ids, pos), cp, "striped", stripe, window=window)
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, window=window)
    compare(o, lse, ro, rl, "bf16", f"all-gather striped({stripe}) cp{cp} window {window}")


def test_allgather_dual_chunk_and_subset_of_ranks():
    """Any reorder works; ranks not run leave their shard of the buffers as it was."""
    ids, pos = packed_metadata(1, 2048, 2, 900)
    q, k, v = random_qkv(1, 2048, 2048, 8, 8, 64, "bf16", seed=22)
    qd, kd, vd, idd, pod = _dev(q, k, v, ids, pos)
    o, lse = bosf.allgather_forward(qd, kd, vd, idd, pod, 4, "dual_chunk", 1, window=(100, 0))
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, window=(100, 0))
    compare(o, lse, ro, rl, "bf16", "all-gather dual chunk")
    bufs = bosf.RingBuffers.like(qd, kd, idd, 4, partials=False)
    bufs.o.fill_(7.0)
    o2, _ = bosf.allgather_forward(qd, kd, vd, idd, pod, 4, "dual_chunk", 1, window=(100, 0),
                                   ranks=[1], bufs=bufs)
    n = 2048 // 4
    assert torch.equal(bufs.o[:, n:2 * n], o2[:, oracle.reorder_map(2048, 4, "dual_chunk", 1)[n:2 * n]])
    assert (bufs.o[:, :n] == 7.0).all() and (bufs.o[:, 2 * n:] == 7.0).all()


def _longctx_allgather():
    return dataclasses.replace(get(5), reorder="striped", stripe=512)


def test_allgather_full_size_sampled():
    """The long-context workload under all-gather CP (striped 512, 4 ranks):
    sampled rows (segment starts, window edges, padding, stripe and shard
    boundaries, random) against the oracle, every head."""
    w = _longctx_allgather()
    q, k, v, ids, pos = device_inputs(w)
    o, lse = bosf.allgather_forward(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe,
                                    causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    left = w.window[0]
    edges = [0, 1, 63, 64, 511, 512, 513, left - 1, left, left + 1, w.valid_per_slot - 1,
             w.valid_per_slot, w.slot_len - 1]
    rows = sample_rows(w, rng, edges)
    m = oracle.reorder_map(w.seq_len, w.cp_size, w.reorder, w.stripe)
    n = w.seq_len // w.cp_size
    for r in range(1, w.cp_size):
        for p in (r * n - 1, r * n):
            rows.append((1, int(m[p])))
    ro, rl = oracle.attention_rows(q, k.cpu(), v.cpu(), ids.cpu(), pos.cpu(), ids.cpu(), pos.cpu(),
                                   rows, causal=w.causal, window=w.window)
    bi = torch.tensor([r[0] for r in rows])
    ti = torch.tensor([r[1] for r in rows])
    e = compare(o[bi, ti], lse[bi, ti], ro, rl, "bf16", "all-gather long context")
    print(f"all-gather long context: {len(rows)} rows x {w.num_q_heads} heads: "
          f"max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")


def test_allgather_full_size_zero_queries_every_row():
    """Q = 0 at full size: LSE = ln(visible keys) on every row and head."""
    w = _longctx_allgather()
    q, k, v, ids, pos = device_inputs(w, zero_q=True)
    o, lse = bosf.allgather_forward(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe,
                                    causal=w.causal, window=w.window)
    nvis = closed_form_counts(w, pos, ids)
    ref = torch.where(nvis > 0, torch.log(nvis), torch.full_like(nvis, -np.inf))
    got = lse.to(torch.float64)
    live = nvis > 0
    assert torch.equal(torch.isneginf(got), ~live[:, :, None].expand_as(got))
    err = (got - ref[:, :, None])[live[:, :, None].expand_as(got)].abs().max().item()
    assert err <= 1e-5, err
    assert (o[~live] == 0).all()


def _plan(w, ids, pos):
    return bosf.ring_plan(ids.to(DEV), pos.to(DEV), w.cp_size, w.reorder, w.stripe,
                          num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim=w.head_dim, causal=w.causal, window=w.window)


def test_ring_plan_counts_match_oracle():
    """Per (rank, step) visible pairs of the sharded packed workload's ring, from
    the library's classification, equal the oracle's mask counts."""
    w = get(3)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    plan = _plan(w, ids, pos).counts
    m = oracle.reorder_map(w.seq_len, w.cp_size, w.reorder, w.stripe)
    ids_r, pos_r = ids.numpy()[:, m], pos.numpy()[:, m]
    n = w.seq_len // w.cp_size
    for r in range(w.cp_size):
        for s in range(w.cp_size):
            c = (r - s) % w.cp_size
            want = oracle.visible_pairs(ids_r[:, r * n:(r + 1) * n], pos_r[:, r * n:(r + 1) * n],
                                        ids_r[:, c * n:(c + 1) * n], pos_r[:, c * n:(c + 1) * n],
                                        causal=w.causal, window=w.window).sum()
            assert int(plan[r, s]) == int(want), (r, s, int(plan[r, s]), int(want))
    assert (plan == 0).any(), "the layout should have empty ring steps"


def test_ring_plan_long_context_total():
    """The long-context ring's plan sums to the step's visible pairs (closed
    form, tests/golden/visible_pairs.txt) and is the same for ranks r and r+2
    (the dual-chunk layout is periodic with period 2 in the rank here)."""
    w = get(5)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    plan = _plan(w, ids, pos).counts
    assert int(plan.sum()) == 536936448
    assert torch.equal(plan[0], plan[2]) and torch.equal(plan[1], plan[3])
    assert (plan == 0).sum() == 8


def test_ring_with_plan_is_bit_identical():
    """Skipping the steps without visible pairs changes nothing: the last
    step that has work writes the same bf16 output the empty step would have."""
    w = dataclasses.replace(get(5), batch=1, seq_len=16384, num_q_heads=16, slots=2,
                            valid_per_slot=6000, window=(2048, 0))
    q, k, v, ids, pos = device_inputs(w)
    plan = bosf.ring_plan(ids, pos, w.cp_size, w.reorder, w.stripe, num_q_heads=w.num_q_heads,
                          num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, causal=w.causal,
                          window=w.window)
    assert (plan.counts == 0).any()
    o1, l1 = bosf.ring_forward(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe,
                               causal=w.causal, window=w.window)
    o2, l2 = bosf.ring_forward(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe,
                               causal=w.causal, window=w.window, plan=plan)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kind", ["dual_chunk", "striped"])
def test_ring_repeated_calls_reuse_plan_schedules(kind):
    """A plan keeps the device schedules of its ring's calls: a second ring_forward
    with the same plan and buffers skips the classification and gives the same
    bits; each call packs its K/V chunks anew, so new K/V values in the same
    buffers give the result of a fresh run."""
    b, t, hq, hkv = 2, 4096, 8, 2
    ids, pos = _dev(*packed_metadata(b, t, 2, 1500))
    q, k, v = _dev(*random_qkv(b, t, t, hq, hkv, 128, "bf16", seed=91))
    kw = dict(causal=True, window=(700, 0))
    halves = kind == "dual_chunk"
    plan = bosf.ring_plan(ids, pos, 4, kind, 1, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                          halves=halves, **kw)
    bufs = bosf.RingBuffers.like(q, k, ids, 4, v=v)
    o1, l1 = bosf.ring_forward(q, k, v, ids, pos, 4, kind, 1, bufs=bufs, plan=plan, **kw)
    o1, l1 = o1.clone(), l1.clone()
    assert plan.ready and plan.ready == set(plan.schedules)
    o2, l2 = bosf.ring_forward(q, k, v, ids, pos, 4, kind, 1, bufs=bufs, plan=plan, **kw)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o0, l0 = bosf.ring_forward(q, k, v, ids, pos, 4, kind, 1, **kw)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    k2, v2 = (k * 0.5).contiguous(), v.flip(1).contiguous()
    o3, l3 = bosf.ring_forward(q, k2, v2, ids, pos, 4, kind, 1, bufs=bufs, plan=plan, **kw)
    o4, l4 = bosf.ring_forward(q, k2, v2, ids, pos, 4, kind, 1, **kw)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    assert not torch.equal(o3, o1)


@pytest.mark.parametrize("cp,window,dtype", [(4, (2048, 0), "bf16"), (2, (-1, -1), "bf16"),
                                             (8, (300, 0), "bf16"), (4, (500, 0), "f32")])
def test_ring_inverse_folded_into_last_step_is_bit_identical(cp, window, dtype):
    """The dual-chunk inverse reorder folded into each rank's last ring step
    (a split output writing O and the LSE at their original positions) gives
    the same bits as the separate inverse-reorder pass, with and without the
    plan of steps, and with the per-stripe plan (each stripe finished at its
    own last step with work)."""
    b, t, hq, hkv = 2, 4096, 8, 2
    ids, pos = packed_metadata(b, t, 2, 1500)
    q, k, v = _dev(*random_qkv(b, t, t, hq, hkv, 64, dtype, seed=cp * 7 + 1))
    ids, pos = _dev(ids, pos)
    kw = dict(causal=True, window=window)
    o_a, l_a = bosf.ring_forward(q, k, v, ids, pos, cp, "dual_chunk", 1, fuse_inverse=False, **kw)
    o_b, l_b = bosf.ring_forward(q, k, v, ids, pos, cp, "dual_chunk", 1, **kw)
    plan = bosf.ring_plan(ids, pos, cp, "dual_chunk", 1, num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=64, dtype=q.dtype, **kw)
    o_c, l_c = bosf.ring_forward(q, k, v, ids, pos, cp, "dual_chunk", 1, plan=plan, **kw)
    hplan = bosf.ring_plan(ids, pos, cp, "dual_chunk", 1, num_q_heads=hq, num_kv_heads=hkv,
                           head_dim=64, dtype=q.dtype, halves=True, **kw)
    assert torch.equal(hplan.counts.sum(1), plan.counts)
    o_d, l_d = bosf.ring_forward(q, k, v, ids, pos, cp, "dual_chunk", 1, plan=hplan, **kw)
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    assert torch.equal(o_a, o_c) and torch.equal(l_a, l_c)
    assert torch.equal(o_a, o_d) and torch.equal(l_a, l_d)
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), ids.cpu(), pos.cpu(), ids.cpu(),
                              pos.cpu(), **kw)
    compare(o_b, l_b, ro, rl, dtype, f"folded inverse cp={cp}")


@pytest.mark.parametrize("dtype,out_dtype", [("bf16", torch.bfloat16), ("bf16", torch.float32),
                                             ("f32", torch.float32)])
def test_split_output_places_rows_and_leaves_the_gap(dtype, out_dtype):
    """attn_fwd and attn_fwd_accumulate with a split output write rows below the
    split at ``out`` and the rest ``o_split_offset`` further on, bit-identical to
    the unsplit call; the gap between them keeps its contents."""
    b, tq, tk, hq, hkv, d, row, gap = 2, 300, 260, 8, 2, 64, 97, 41
    rng = np.random.default_rng(3)
    from workloads import random_layout
    qi, qp = random_layout(rng, b, tq, max_segments=3, pad_prob=0.2, pos_offset_max=5)
    ki, kp = random_layout(rng, b, tk, max_segments=3, pad_prob=0.2, pos_offset_max=40)
    q, k, v = _dev(*random_qkv(b, tq, tk, hq, hkv, d, dtype, seed=11))
    qi, qp, ki, kp = _dev(qi, qp, ki, kp)
    kw = dict(causal=True, window=(120, 0), out_dtype=out_dtype)
    o_ref, l_ref = bosf.attn_fwd(q, k, v, qi, qp, ki, kp, **kw)
    big_o = torch.full((b, tq + gap, hq, d), 7.0, dtype=out_dtype, device=DEV)
    big_l = torch.full((b, tq + gap, hq), 7.0, dtype=torch.float32, device=DEV)
    bosf.attn_fwd(q, k, v, qi, qp, ki, kp, out=big_o[:, :row], lse=big_l[:, :row],
                  split=(row, big_o[:, row + gap:], big_l[:, row + gap:]), **kw)
    assert torch.equal(big_o[:, :row], o_ref[:, :row]) and torch.equal(big_o[:, row + gap:], o_ref[:, row:])
    assert torch.equal(big_l[:, :row], l_ref[:, :row]) and torch.equal(big_l[:, row + gap:], l_ref[:, row:])
    assert (big_o[:, row:row + gap] == 7.0).all() and (big_l[:, row:row + gap] == 7.0).all()
    # accumulate: fold the second half of the keys into the first half's partial
    h = tk // 2
    po, pl = bosf.attn_fwd(q, k[:, :h], v[:, :h], qi, qp, ki[:, :h], kp[:, :h], causal=True,
                           window=(120, 0), out_dtype=torch.float32)
    ref_o, ref_l = bosf.attn_fwd_accumulate(q, k[:, h:], v[:, h:], qi, qp, ki[:, h:], kp[:, h:],
                                            po.clone(), pl.clone(), causal=True, window=(120, 0),
                                            out=torch.empty_like(o_ref), lse=torch.empty_like(l_ref))
    big_o.fill_(7.0)
    big_l.fill_(7.0)
    bosf.attn_fwd_accumulate(q, k[:, h:], v[:, h:], qi, qp, ki[:, h:], kp[:, h:], po, pl,
                             causal=True, window=(120, 0), out=big_o[:, :row], lse=big_l[:, :row],
                             split=(row, big_o[:, row + gap:], big_l[:, row + gap:]))
    assert torch.equal(big_o[:, :row], ref_o[:, :row]) and torch.equal(big_o[:, row + gap:], ref_o[:, row:])
    assert torch.equal(big_l[:, :row], ref_l[:, :row]) and torch.equal(big_l[:, row + gap:], ref_l[:, row:])
    assert (big_o[:, row:row + gap] == 7.0).all() and (big_l[:, row:row + gap] == 7.0).all()
