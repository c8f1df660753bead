"""GPU parity of the attention backward against the fp64 backward oracle.

The HIP path gets o and lse from the library's own forward (as a caller
would), then dq, dk and dv from ``attn_bwd``; the oracle differentiates the
plain masked softmax attention in fp64 from the same q, k, v and dout.  Small
cases cover every GQA group size, both head dims, windows at their edges,
cross-attention with unrelated layouts, ragged tails of both tile shapes,
o in bf16 and fp32, gradients in fp32 and bf16, batch-strided views and empty
inputs, compared element by element.  At full size the packed GQA workload is
compared everywhere; the larger workloads on sampled query rows, on keys
whose gradient the oracle can form quickly (the ends of segments and of the
sequence, padding), and on identities that hold for every key: per segment
and K/V head, the keys' dK sum to 0 (softmax ignores a common shift of the
scores) and their dV sum to the sum of the live queries' dO (each row of P
sums to 1).  With Q = 0 every probability is 1/n, so dV has a closed form on
every key.
"""

import dataclasses

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare_grads
from _workload_io import closed_form_counts, device_inputs
from workloads import get, random_layout, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _fwd_bwd(q, k, v, qi, qp, ki, kp, do, causal, window, o_dtype=None, grad_dtype=torch.float32):
    o, lse = bosf.attn_fwd(q, k, v, qi, qp, ki, kp, causal=causal, window=window,
                           out_dtype=o_dtype)
    return bosf.attn_bwd(q, k, v, qi, qp, ki, kp, o, lse, do, causal=causal, window=window,
                         grad_dtype=grad_dtype)


def _unreached(qi, qp, ki, kp, causal, window):
    """Masks of query rows and key rows that no visible pair reaches."""
    vis = np.stack([oracle.visible(qi[b], qp[b], ki[b], kp[b], causal, window)
                    for b in range(qi.shape[0])])
    return ~vis.any(axis=2), ~vis.any(axis=1)


# (B, Tq, Tk, Hq, Hkv, D, causal, window, self_attention)
SMALL = [
    (1, 1, 1, 1, 1, 64, True, (-1, -1), True),
    (1, 33, 33, 8, 8, 128, True, (-1, -1), True),
    (2, 257, 257, 16, 2, 128, True, (-1, -1), True),
    (2, 300, 300, 16, 2, 128, True, (40, 0), True),
    (1, 517, 517, 64, 8, 128, True, (100, 0), True),
    (2, 200, 200, 32, 2, 128, True, (0, 0), True),
    (2, 190, 190, 4, 1, 64, False, (-1, -1), True),
    (1, 250, 250, 8, 4, 64, False, (17, 9), True),
    (2, 129, 129, 3, 1, 128, True, (-1, 5), True),
    (1, 300, 300, 12, 1, 128, True, (-1, -1), True),
    (2, 161, 161, 6, 3, 64, True, (30, 30), True),
    (1, 96, 96, 1, 1, 128, True, (-1, -1), True),
    (2, 300, 517, 16, 2, 128, True, (-1, -1), False),
    (1, 517, 300, 8, 2, 64, False, (50, 50), False),
    (2, 64, 640, 16, 1, 128, True, (200, 0), False),
    (1, 700, 45, 4, 2, 128, False, (-1, -1), False),
    # dK/dV pass: 45 key-tile items in runs of 6, later keys seen by more
    # queries (window (0, -1)), so runs are dealt in reverse, the last one
    # with 3 items and 3 positions past the end
    (5, 2304, 2304, 8, 1, 64, False, (0, -1), True),
]


def _case_id(c):
    b, tq, tk, hq, hkv, d, causal, w, self_ = c
    return (f"B{b}_Tq{tq}_Tk{tk}_H{hq}-{hkv}_D{d}_{'c' if causal else 'nc'}_w{w[0]}.{w[1]}_"
            f"{'self' if self_ else 'cross'}")


def _small_inputs(case):
    b, tq, tk, hq, hkv, d, causal, window, self_ = case
    rng = np.random.default_rng(tq * 11 + tk + hq)
    qi, qp = random_layout(rng, b, tq, max_segments=4, pad_prob=0.25, pos_offset_max=3)
    if self_:
        ki, kp = qi, qp
    else:
        ki, kp = random_layout(rng, b, tk, max_segments=3, pad_prob=0.25, pos_offset_max=40)
    q, k, v = random_qkv(b, tq, tk, hq, hkv, d, "bf16", seed=tq + 3 * tk)
    do = random_qkv(b, tq, 1, hq, 1, d, "bf16", seed=tq + 5 * tk + 1)[0]
    return q, k, v, do, qi, qp, ki, kp


def test_negative_segment_ids():
    """Segment ids of either sign (0 marks padding): a padding query never sees
    a key of id -1 and no query sees a padding key, in both passes."""
    rng = np.random.default_rng(74)
    ids, pos = random_layout(rng, 2, 300, max_segments=6, pad_prob=0.4, pos_offset_max=3)
    ids = torch.where(ids != 0, -ids, ids)
    assert (ids == -1).any() and (ids == 0).any()
    q, k, v = random_qkv(2, 300, 300, 16, 2, 128, "bf16", seed=75)
    do = random_qkv(2, 300, 1, 16, 1, 128, "bf16", seed=76)[0]
    for causal, window in ((True, (50, 0)), (False, (-1, -1))):
        dq, dk, dv = _fwd_bwd(*_dev(q, k, v, ids, pos, ids, pos, do), causal, window)
        torch.cuda.synchronize()
        refs = oracle.attention_backward(q, k, v, do, ids, pos, ids, pos, causal=causal,
                                         window=window)
        zq, zk = _unreached(ids.numpy(), pos.numpy(), ids.numpy(), pos.numpy(), causal, window)
        for got, ref, z, name in ((dq, refs[0], zq, "dq"), (dk, refs[1], zk, "dk"),
                                  (dv, refs[2], zk, "dv")):
            compare_grads(got, ref, f"negative ids causal={causal} {name}",
                          exact_zero=np.broadcast_to(z[:, :, None, None], ref.shape))


@pytest.mark.parametrize("case", SMALL, ids=[_case_id(c) for c in SMALL])
@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
def test_small_random_layouts(case, o_dtype):
    causal, window = case[6], case[7]
    q, k, v, do, qi, qp, ki, kp = _small_inputs(case)
    od = torch.float32 if o_dtype == "f32" else None
    dq, dk, dv = _fwd_bwd(*_dev(q, k, v, qi, qp, ki, kp, do), causal, window, od)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, causal=causal, window=window)
    zq, zk = _unreached(qi.numpy(), qp.numpy(), ki.numpy(), kp.numpy(), causal, window)
    what = f"{_case_id(case)} o {o_dtype}"
    compare_grads(dq, rq, what + " dq", exact_zero=np.broadcast_to(zq[:, :, None, None], rq.shape))
    compare_grads(dk, rk, what + " dk", exact_zero=np.broadcast_to(zk[:, :, None, None], rk.shape))
    compare_grads(dv, rv, what + " dv", exact_zero=np.broadcast_to(zk[:, :, None, None], rv.shape))


@pytest.mark.parametrize("case", [SMALL[3], SMALL[7], SMALL[12]], ids=lambda c: _case_id(c))
def test_bf16_gradients(case):
    causal, window = case[6], case[7]
    q, k, v, do, qi, qp, ki, kp = _small_inputs(case)
    dq, dk, dv = _fwd_bwd(*_dev(q, k, v, qi, qp, ki, kp, do), causal, window,
                          grad_dtype=torch.bfloat16)
    assert dq.dtype == dk.dtype == dv.dtype == torch.bfloat16
    rq, rk, rv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, causal=causal, window=window)
    for got, ref, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        compare_grads(got, ref, f"{_case_id(case)} bf16 {n}")


def test_strided_views_and_determinism():
    """Shards of larger buffers (batch stride above the dense value) in and out,
    and two calls giving bit-identical gradients (no atomics)."""
    b, tq, tk, hq, hkv, d = 2, 200, 330, 8, 2, 128
    rng = np.random.default_rng(5)
    qi, qp = random_layout(rng, b, tq, max_segments=3, pad_prob=0.2)
    ki, kp = random_layout(rng, b, tk, max_segments=2, pad_prob=0.2, pos_offset_max=50)
    q, k, v = random_qkv(b, tq, tk, hq, hkv, d, "bf16", seed=77)
    do = random_qkv(b, tq, 1, hq, 1, d, "bf16", seed=78)[0]
    big_q = torch.zeros((b, tq + 64, hq, d), dtype=torch.bfloat16, device=DEV)
    big_k = torch.zeros((b, tk + 32, hkv, d), dtype=torch.bfloat16, device=DEV)
    big_v = torch.zeros_like(big_k)
    big_do = torch.zeros_like(big_q)
    qv, kv_, vv, dov = big_q[:, 64:], big_k[:, :tk], big_v[:, :tk], big_do[:, 64:]
    qv.copy_(q.to(DEV)); kv_.copy_(k.to(DEV)); vv.copy_(v.to(DEV)); dov.copy_(do.to(DEV))
    mi = _dev(qi, qp, ki, kp)
    big_o = torch.zeros((b, tq + 64, hq, d), dtype=torch.bfloat16, device=DEV)
    o, lse = bosf.attn_fwd(qv, kv_, vv, *mi, out=big_o[:, 64:])
    gq = torch.full((b, tq + 64, hq, d), 7.0, device=DEV)
    gk = torch.full((b, tk + 32, hkv, d), 7.0, device=DEV)
    gv = torch.full((b, tk + 32, hkv, d), 7.0, device=DEV)
    dq, dk, dv = bosf.attn_bwd(qv, kv_, vv, *mi, o, lse, dov, dq=gq[:, 64:], dk=gk[:, :tk],
                               dv=gv[:, :tk])
    assert (gq[:, :64] == 7.0).all() and (gk[:, tk:] == 7.0).all() and (gv[:, tk:] == 7.0).all()
    rq, rk, rv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp)
    compare_grads(dq, rq, "strided dq")
    compare_grads(dk, rk, "strided dk")
    compare_grads(dv, rv, "strided dv")
    dq2, dk2, dv2 = bosf.attn_bwd(qv, kv_, vv, *mi, o, lse, dov)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_empty_and_unreachable():
    """Empty lengths, all-padding rows and disjoint segments give exact zeros."""
    d = 128
    for tq, tk in ((0, 64), (64, 0), (0, 0)):
        q = torch.zeros((1, tq, 4, d), dtype=torch.bfloat16, device=DEV)
        k = torch.zeros((1, tk, 2, d), dtype=torch.bfloat16, device=DEV)
        qi = torch.ones((1, tq), dtype=torch.int32, device=DEV)
        ki = torch.ones((1, tk), dtype=torch.int32, device=DEV)
        o, lse = bosf.attn_fwd(q, k, k, qi, qi, ki, ki)
        dq, dk, dv = bosf.attn_bwd(q, k, k, qi, qi, ki, ki, o, lse, q)
        torch.cuda.synchronize()
        assert dq.shape == q.shape and dk.shape == k.shape
        assert not dq.any() and not dk.any() and not dv.any()
    # queries and keys in different segments, plus an all-padding batch row
    b, tq, tk, hq, hkv = 2, 150, 170, 8, 2
    q, k, v = random_qkv(b, tq, tk, hq, hkv, d, "bf16", seed=3, device=DEV)
    do = random_qkv(b, tq, 1, hq, 1, d, "bf16", seed=4, device=DEV)[0]
    qi = torch.full((b, tq), 1, dtype=torch.int32, device=DEV)
    ki = torch.full((b, tk), 2, dtype=torch.int32, device=DEV)
    qi[1] = 0
    pos_q = torch.arange(tq, dtype=torch.int32, device=DEV).expand(b, tq).contiguous()
    pos_k = torch.arange(tk, dtype=torch.int32, device=DEV).expand(b, tk).contiguous()
    o, lse = bosf.attn_fwd(q, k, v, qi, pos_q, ki, pos_k, causal=False)
    dq, dk, dv = bosf.attn_bwd(q, k, v, qi, pos_q, ki, pos_k, o, lse, do, causal=False)
    torch.cuda.synchronize()
    assert not dq.any() and not dk.any() and not dv.any()


# ----------------------------------------------------------------------------- full size


def _device_do(w, shape, seed_off=17):
    g = torch.Generator(device=DEV)
    g.manual_seed(w.seed + seed_off)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


def _segment_identities(dk, dv, do, q_ids, k_ids, group, what, tol=1e-2):
    """Per batch row, segment and K/V head: sum_j dK_j = 0 and sum_j dV_j =
    sum over live queries and the group's heads of dO, each measured against the
    root-sum-square of the terms (the size of the summed rounding errors)."""
    dk64, dv64 = dk.to(torch.float64), dv.to(torch.float64)
    do64 = do.to(torch.float64)
    b_, tq, hq, d = do.shape
    hkv = dk.shape[2]
    worst = [0.0, 0.0]
    for b in range(b_):
        for sid in torch.unique(k_ids[b]).tolist():
            if sid == 0:
                continue
            ks = k_ids[b] == sid
            qs = q_ids[b] == sid
            sk = dk64[b, ks].sum(0)                                # [Hkv, D]
            rk = dk64[b, ks].pow(2).sum(0).sum(-1).sqrt()          # [Hkv]
            sv = dv64[b, ks].sum(0)
            rv = dv64[b, ks].pow(2).sum(0).sum(-1).sqrt()
            want = do64[b, qs].reshape(-1, hkv, group, d).sum(dim=(0, 2))
            ek = (sk.norm(dim=-1) / rk.clamp_min(1e-30)).max().item()
            ev = ((sv - want).norm(dim=-1) / rv.clamp_min(1e-30)).max().item()
            worst = [max(worst[0], ek), max(worst[1], ev)]
    assert worst[0] <= tol, f"{what}: |sum dK| / rss(dK) = {worst[0]:.3e}"
    assert worst[1] <= tol, f"{what}: |sum dV - sum dO| / rss(dV) = {worst[1]:.3e}"
    return worst


def test_packed_gqa_full_size_everywhere():
    """The packed GQA workload (2 x 4096 tokens, 16/2 heads, causal, padding):
    every gradient element against the oracle."""
    w = get(2)
    q, k, v, ids, pos = device_inputs(w)
    do = _device_do(w, q.shape)
    dq, dk, dv = _fwd_bwd(q, k, v, ids, pos, ids, pos, do, w.causal, w.window)
    torch.cuda.synchronize()
    idc, poc = ids.cpu(), pos.cpu()
    rq, rk, rv = oracle.attention_backward(q.cpu(), k.cpu(), v.cpu(), do.cpu(), idc, poc, idc, poc,
                                           causal=w.causal, window=w.window)
    pad = (idc == 0).numpy()[:, :, None, None]
    res = [compare_grads(dq, rq, "packed gqa dq", exact_zero=np.broadcast_to(pad, rq.shape)),
           compare_grads(dk, rk, "packed gqa dk", exact_zero=np.broadcast_to(pad, rk.shape)),
           compare_grads(dv, rv, "packed gqa dv", exact_zero=np.broadcast_to(pad, rv.shape))]
    print("packed gqa full size (rel fro, max/max|ref|):", res)


def _sampled_check(w, q, k, v, ids_q, pos_q, ids_k, pos_k, do, dq, dk, dv, q_rows, k_rows, what):
    kw = dict(causal=w.causal, window=w.window)
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    iq, pq, ik, pk = ids_q.cpu(), pos_q.cpu(), ids_k.cpu(), pos_k.cpu()
    rq = oracle.backward_query_rows(qc, kc, vc, doc, iq, pq, ik, pk, q_rows, **kw)
    bi = torch.tensor([r[0] for r in q_rows])
    ti = torch.tensor([r[1] for r in q_rows])
    e1 = compare_grads(dq[bi, ti], rq, what + " sampled dq")
    rk, rv = oracle.backward_key_rows(qc, kc, vc, doc, iq, pq, ik, pk, k_rows, **kw)
    bi = torch.tensor([r[0] for r in k_rows])
    ti = torch.tensor([r[1] for r in k_rows])
    e2 = compare_grads(dk[bi, ti], rk, what + " sampled dk")
    e3 = compare_grads(dv[bi, ti], rv, what + " sampled dv")
    return e1, e2, e3


def _end_keys(w, extra=()):
    """Keys at the ends of segments (few queries see them) and padding keys."""
    keys = []
    for b in range(w.batch):
        for s in range(w.slots):
            base = s * w.slot_len
            for p in (w.valid_per_slot - 1, w.valid_per_slot - 2, w.valid_per_slot - 40):
                keys.append((b, base + p))
            if w.valid_per_slot < w.slot_len:
                keys.append((b, base + w.valid_per_slot))          # padding
    return sorted(set(keys) | set(extra))


def test_swa_full_size_sampled_and_identities():
    """Causal sliding window GQA (32768 tokens, 64/8 heads, window 4096)."""
    w = get(4)
    q, k, v, ids, pos = device_inputs(w)
    do = _device_do(w, q.shape)
    dq, dk, dv = _fwd_bwd(q, k, v, ids, pos, ids, pos, do, w.causal, w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    rows = sorted({(0, int(t)) for t in list(rng.integers(0, w.seq_len, 24)) +
                   [0, 1, 63, 64, 4095, 4096, 4097, w.seq_len - 1]})
    e = _sampled_check(w, q, k, v, ids, pos, ids, pos, do, dq, dk, dv, rows, _end_keys(w), "swa")
    ident = _segment_identities(dk, dv, do, ids, ids, w.group, "swa")
    print("swa sampled:", e, "identities:", ident)


def _longctx_allgather_shard():
    """Rank 1's share of the long-context workload under all-gather CP (striped
    512 reorder): its 16384-token query shard per row against all 65536 keys."""
    w = dataclasses.replace(get(5), reorder="striped", stripe=512)
    q, k, v, ids, pos = device_inputs(w)
    m = torch.from_numpy(oracle.reorder_map(w.seq_len, w.cp_size, w.reorder, w.stripe)).long().to(DEV)
    q, k, v, ids, pos = (t[:, m].contiguous() for t in (q, k, v, ids, pos))
    n = w.seq_len // w.cp_size
    r = 1
    sl = slice(r * n, (r + 1) * n)
    return w, q[:, sl].contiguous(), k, v, ids[:, sl].contiguous(), pos[:, sl].contiguous(), ids, pos


def test_longctx_allgather_shard_sampled_and_identities():
    w, q, k, v, iq, pq, ik, pk = _longctx_allgather_shard()
    do = _device_do(w, q.shape)
    dq, dk, dv = _fwd_bwd(q, k, v, iq, pq, ik, pk, do, w.causal, w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(51)
    rows = sorted({(int(rng.integers(0, w.batch)), int(rng.integers(0, q.shape[1])))
                   for _ in range(24)} | {(0, 0), (1, q.shape[1] - 1), (0, 511), (0, 512)})
    # Keys that only the shard's last queries of a segment see (cheap for the
    # oracle, and nonzero), keys no query of the shard sees (exact 0), and
    # padding keys, located in the reordered K/V.
    iqc, pqc = iq.cpu().numpy(), pq.cpu().numpy()
    ikc, pkc = ik.cpu().numpy(), pk.cpu().numpy()
    keys = []
    for b in range(w.batch):
        for sid in np.unique(iqc[b]):
            if sid == 0:
                continue
            pmax = int(pqc[b][iqc[b] == sid].max())
            for p in (pmax, pmax - 1, pmax - 33, pmax + 1):
                hits = np.nonzero((ikc[b] == sid) & (pkc[b] == p))[0]
                keys += [(b, int(j)) for j in hits[:1]]
        keys += [(b, int(j)) for j in np.nonzero(ikc[b] == 0)[0][:2]]
    e = _sampled_check(w, q, k, v, iq, pq, ik, pk, do, dq, dk, dv, rows, sorted(set(keys)),
                       "long-context shard")
    ident = _segment_identities(dk, dv, do, iq, ik, w.group, "long-context shard")
    print("long-context shard sampled:", e, "identities:", ident)


def test_zero_queries_dv_closed_form_every_key():
    """Q = 0 on the causal SWA workload: every visible probability is 1/n_i, so
    dK = 0 and dV_j = sum over heads of the group and over the queries i that
    see key j of dO_i / n_i, on every key (windowed prefix sums in fp64)."""
    w = get(4)
    q, k, v, ids, pos = device_inputs(w, zero_q=True)
    do = _device_do(w, q.shape)
    dq, dk, dv = _fwd_bwd(q, k, v, ids, pos, ids, pos, do, w.causal, w.window)
    torch.cuda.synchronize()
    assert dk.abs().max().item() <= 1e-6 * max(1.0, dv.abs().max().item())
    n = closed_form_counts(w, pos[0], ids[0])                       # [T] visible keys per query
    c = do[0].to(torch.float64).reshape(w.seq_len, w.num_kv_heads, w.group, w.head_dim).sum(2)
    c = c / n[:, None, None]
    pref = torch.cat([torch.zeros_like(c[:1]), c.cumsum(0)])        # pref[i] = sum_{t < i}
    t = torch.arange(w.seq_len, device=DEV)
    hi = torch.clamp(t + w.window[0] + 1, max=w.seq_len)            # queries t..t+left see key t
    want = pref[hi] - pref[t]
    got = dv[0].to(torch.float64)
    err = ((got - want).norm() / want.norm()).item()
    mx = ((got - want).abs().max() / want.abs().max()).item()
    print(f"Q=0 dV closed form: rel fro {err:.3e}, max {mx:.3e}")
    assert err <= 1e-2 and mx <= 2e-2
