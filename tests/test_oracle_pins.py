"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes part of the oracle with something independent of its own code:
a library routine (torch's CPU scaled-dot-product attention in fp64), closed
forms of the workloads' masks, exact special cases (uniform V, a single
visible key, zero queries), invariants of the online-softmax merge ("Context
parallelism and ring attention", section "Online softmax"), scalar brute force
with ``math.fsum`` on tiny inputs, hand-worked reorder maps and the interval
geometry of causal / windowed tiles.  Plausible slips in the oracle -- a
dropped mask term, an off-by-one window, a wrong GQA head index, a transposed
operand, log2 instead of ln, a lost scale -- each fail at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import packed_metadata, random_layout, random_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(t):
    return t.to(torch.float64).numpy()


def _contig_meta(batch, t):
    ids = torch.ones(batch, t, dtype=torch.int32)
    pos = torch.arange(t, dtype=torch.int32)[None, :].repeat(batch, 1)
    return ids, pos


# --------------------------------------------------------------------------- library pin

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 1)])
def test_matches_torch_sdpa_fp64(causal, hq, hkv):
    """One unpadded segment, positions 0..T-1: the mask reduces to none or the
    plain causal triangle, which torch's SDPA implements (GQA by head groups)."""
    b, t, d = 2, 37, 16
    q, k, v = random_qkv(b, t, t, hq, hkv, d, "f32", seed=11)
    ids, pos = _contig_meta(b, t)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=causal)
    ref = F.scaled_dot_product_attention(
        q.double().transpose(1, 2), k.double().transpose(1, 2), v.double().transpose(1, 2),
        is_causal=causal, enable_gqa=True).transpose(1, 2).numpy()
    assert np.abs(o - ref).max() < 1e-12
    assert np.isfinite(lse).all()


def test_sdpa_scale_is_head_dim_rsqrt():
    """The default scale is head_dim**-0.5 (tutorial section 3, scaling_factor)."""
    b, t, d = 1, 20, 32
    q, k, v = random_qkv(b, t, t, 2, 2, d, "f32", seed=5)
    ids, pos = _contig_meta(b, t)
    o, _ = oracle.attention(q, k, v, ids, pos, ids, pos, causal=False)
    ref = F.scaled_dot_product_attention(
        q.double().transpose(1, 2), k.double().transpose(1, 2), v.double().transpose(1, 2),
        scale=d ** -0.5).transpose(1, 2).numpy()
    assert np.abs(o - ref).max() < 1e-12
    o2, _ = oracle.attention(q, k, v, ids, pos, ids, pos, causal=False, scale=0.3)
    ref2 = F.scaled_dot_product_attention(
        q.double().transpose(1, 2), k.double().transpose(1, 2), v.double().transpose(1, 2),
        scale=0.3).transpose(1, 2).numpy()
    assert np.abs(o2 - ref2).max() < 1e-12


@pytest.mark.parametrize("d,dv,causal", [(24, 16, True), (12, 20, False)])
def test_value_head_dim_differs_torch_sdpa(d, dv, causal):
    """V's head dim differing from Q/K's (MLA head dimensions, tutorial's
    "Next steps"): torch's SDPA in fp64 takes the same shapes; scale D**-0.5."""
    b, t, hq, hkv = 2, 29, 4, 2
    q, k, _ = random_qkv(b, t, t, hq, hkv, d, "f32", seed=21)
    v = random_qkv(b, t, t, hq, hkv, dv, "f32", seed=22)[2]
    ids, pos = _contig_meta(b, t)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=causal)
    assert o.shape == (b, t, hq, dv)
    ref = F.scaled_dot_product_attention(
        q.double().transpose(1, 2), k.double().transpose(1, 2), v.double().transpose(1, 2),
        is_causal=causal, enable_gqa=True).transpose(1, 2).numpy()
    assert np.abs(o - ref).max() < 1e-12
    rows = [(0, 0), (1, 17), (1, 28)]
    o2, l2 = oracle.attention_rows(q, k, v, ids, pos, ids, pos, rows, causal=causal)
    for n, (bb, i) in enumerate(rows):
        assert np.abs(o2[n] - o[bb, i]).max() < 1e-13 and np.abs(l2[n] - lse[bb, i]).max() < 1e-13


# --------------------------------------------------------------------------- exact special cases

def _layouts():
    rng = np.random.default_rng(3)
    out = [packed_metadata(2, 96, 4, 18)]
    for _ in range(3):
        out.append(random_layout(rng, 2, 90, max_segments=5, pad_prob=0.3))
    return out


@pytest.mark.parametrize("window", [(-1, -1), (5, 0), (0, 3), (7, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_uniform_v_gives_constant_output(window, causal):
    """P1: with v[b, j, g, :] = c_g the softmax weights sum to one, so every
    row with a visible key returns c_g exactly, and empty rows return 0."""
    for ids, pos in _layouts():
        b, t = ids.shape
        hq, hkv, d = 6, 3, 8
        q, k, _ = random_qkv(b, t, t, hq, hkv, d, "f32", seed=7)
        c = np.random.default_rng(1).normal(size=(hkv, d))
        v = np.broadcast_to(c[None, None], (b, t, hkv, d)).copy()
        o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=causal, window=window)
        for h in range(hq):
            g = h // (hq // hkv)
            live = np.isfinite(lse[:, :, h])
            assert np.abs(o[:, :, h][live] - c[g]).max() < 1e-12
            assert (o[:, :, h][~live] == 0).all()
        # padding queries never see anything
        assert np.isneginf(lse[_f64(ids) == 0]).all()


def test_single_visible_key_returns_that_value():
    """P2a: a causal query at segment position 0 sees only itself: O = v,
    LSE = scale * q.k (the softmax of one element is 1)."""
    ids, pos = packed_metadata(2, 64, 4, 12)
    b, t = ids.shape
    hq, hkv, d = 8, 2, 16
    q, k, v = random_qkv(b, t, t, hq, hkv, d, "bf16", seed=9)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True)
    qn, kn, vn = _f64(q), _f64(k), _f64(v)
    starts = [(bb, i) for bb in range(b) for i in range(t) if pos[bb, i] == 0 and ids[bb, i] != 0]
    assert len(starts) == 8
    for bb, i in starts:
        for h in range(hq):
            g = h // (hq // hkv)
            assert np.array_equal(o[bb, i, h], vn[bb, i, g])
            s = float(np.dot(qn[bb, i, h], kn[bb, i, g])) * d ** -0.5
            assert abs(lse[bb, i, h] - s) < 1e-12


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (16, 1), (12, 4)])
def test_window_zero_sees_only_itself(hq, hkv):
    """P2b: causal with window (0, 0): each valid token sees only itself, so
    O[b,t,h] = V[b,t,h // G] exactly -- this fixes the GQA head pairing."""
    rng = np.random.default_rng(hq * 31 + hkv)
    ids, pos = random_layout(rng, 2, 77, max_segments=4, pad_prob=0.25)
    b, t = ids.shape
    d = 8
    q, k, v = random_qkv(b, t, t, hq, hkv, d, "bf16", seed=hq + hkv)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True, window=(0, 0))
    qn, kn, vn = _f64(q), _f64(k), _f64(v)
    g_of = np.arange(hq) // (hq // hkv)
    valid = _f64(ids) != 0
    for bb in range(b):
        for i in range(t):
            if not valid[bb, i]:
                assert np.isneginf(lse[bb, i]).all() and (o[bb, i] == 0).all()
                continue
            assert np.array_equal(o[bb, i], vn[bb, i, g_of])
            s = np.einsum("hd,hd->h", qn[bb, i], kn[bb, i, g_of]) * d ** -0.5
            assert np.abs(lse[bb, i] - s).max() < 1e-12


@pytest.mark.parametrize("left", [-1, 0, 1, 9, 40])
def test_zero_queries_closed_form(left):
    """P3: Q = 0 makes every visible score 0, so LSE = ln(n_i) and O is the
    mean of the visible V rows.  On the packed layout a valid query at position
    p sees n = min(p + 1, left + 1) keys (p + 1 when unbounded): the keys at
    array indices i-n+1 .. i.  Pins the window's inclusive edge and padding."""
    ids, pos = packed_metadata(2, 120, 3, 31)
    b, t = ids.shape
    hq, hkv, d = 4, 2, 8
    _, k, v = random_qkv(b, t, t, hq, hkv, d, "bf16", seed=21)
    q = torch.zeros(b, t, hq, d)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True, window=(left, 0))
    vn = _f64(v)
    for bb in range(b):
        for i in range(t):
            if ids[bb, i] == 0:
                assert np.isneginf(lse[bb, i]).all()
                continue
            p = int(pos[bb, i])
            n = p + 1 if left < 0 else min(p + 1, left + 1)
            assert np.abs(lse[bb, i] - math.log(n)).max() < 1e-12
            mean = vn[bb, i - n + 1:i + 1].mean(axis=0)          # [Hkv, D]
            ref = mean[np.arange(hq) // (hq // hkv)]
            assert np.abs(o[bb, i] - ref).max() < 1e-12


def test_zero_queries_right_window():
    """P3 for the right edge: non-causal, window (0, r): a valid query at
    position p of a segment of n tokens sees min(r, n - 1 - p) + 1 keys."""
    ids, pos = packed_metadata(1, 60, 2, 25)
    t = ids.shape[1]
    _, k, v = random_qkv(1, t, t, 2, 1, 4, "f32", seed=2)
    q = torch.zeros(1, t, 2, 4)
    for r in (0, 3, 30):
        _, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=False, window=(0, r))
        for i in range(t):
            if ids[0, i] == 0:
                continue
            p = int(pos[0, i])
            n = min(r, 25 - 1 - p) + 1
            assert abs(lse[0, i, 0] - math.log(n)) < 1e-12


# --------------------------------------------------------------------------- merge / fold

def _split_keys(rng, t, parts):
    lab = rng.integers(0, parts, size=t)
    return [np.nonzero(lab == j)[0] for j in range(parts)]


@pytest.mark.parametrize("parts", [2, 3, 5])
def test_merge_of_disjoint_key_blocks_equals_unsplit(parts):
    """P4: attention over a union of disjoint key sets equals the merge of the
    per-set results -- both in the (O, LSE) form and in the page's (m, z, u)
    fold.  Fixes the merge weights, its -inf handling and the LSE's base and
    scale (a wrong LSE mis-weights the blocks)."""
    rng = np.random.default_rng(parts)
    ids, pos = random_layout(rng, 2, 70, max_segments=3, pad_prob=0.2)
    b, t = ids.shape
    q, k, v = random_qkv(b, t, t, 4, 2, 8, "bf16", seed=parts)
    full_o, full_l = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True, window=(20, 0))
    blocks = _split_keys(rng, t, parts)
    acc = None
    state = None
    for sel in blocks:
        o_j, l_j = oracle.attention(q, k[:, sel], v[:, sel], ids, pos, ids[:, sel], pos[:, sel],
                                    causal=True, window=(20, 0))
        acc = (o_j, l_j) if acc is None else oracle.merge(acc[0], acc[1], o_j, l_j)
        st = oracle.state_from_output(o_j, l_j)
        state = st if state is None else oracle.fold_mzu(state, st)
    assert np.abs(acc[0] - full_o).max() < 1e-12
    fin = np.isfinite(full_l)
    assert np.array_equal(np.isneginf(acc[1]), ~fin)
    assert np.abs(acc[1][fin] - full_l[fin]).max() < 1e-12
    fo, fl = oracle.state_to_output(*state)
    assert np.abs(fo - full_o).max() < 1e-12
    assert np.abs(fl[fin] - full_l[fin]).max() < 1e-12


def test_merge_identity_commutative_associative():
    rng = np.random.default_rng(0)
    n, d = 50, 6
    os_ = [rng.normal(size=(n, d)) for _ in range(3)]
    ls = [rng.normal(size=n) * 3 for _ in range(3)]
    for j in range(3):                    # sprinkle empty rows
        e = rng.random(n) < 0.3
        ls[j][e] = -np.inf
        os_[j][e] = 0.0
    zero_o, zero_l = np.zeros((n, d)), np.full(n, -np.inf)
    o, l = oracle.merge(os_[0], ls[0], zero_o, zero_l)
    assert np.array_equal(o, os_[0]) and np.array_equal(l, ls[0])
    o_ab, l_ab = oracle.merge(os_[0], ls[0], os_[1], ls[1])
    o_ba, l_ba = oracle.merge(os_[1], ls[1], os_[0], ls[0])
    assert np.abs(o_ab - o_ba).max() < 1e-14 and np.array_equal(np.isneginf(l_ab), np.isneginf(l_ba))
    o1, l1 = oracle.merge(*oracle.merge(os_[0], ls[0], os_[1], ls[1]), os_[2], ls[2])
    o2, l2 = oracle.merge(os_[0], ls[0], *oracle.merge(os_[1], ls[1], os_[2], ls[2]))
    assert np.abs(o1 - o2).max() < 1e-12
    f = np.isfinite(l1)
    assert np.abs(l1[f] - l2[f]).max() < 1e-12 and np.array_equal(f, np.isfinite(l2))
    assert not np.isnan(o1).any() and not np.isnan(l1).any()


def test_merge_infinity_rules():
    """Reading for rows with no visible key: both empty -> (0, -inf); one
    empty -> the other, unchanged."""
    o_a = np.array([[1.5, -2.0], [0.0, 0.0], [0.0, 0.0]])
    l_a = np.array([0.7, -np.inf, -np.inf])
    o_b = np.array([[0.0, 0.0], [3.0, 4.0], [0.0, 0.0]])
    l_b = np.array([-np.inf, -1.25, -np.inf])
    o, l = oracle.merge(o_a, l_a, o_b, l_b)
    assert np.array_equal(o, np.array([[1.5, -2.0], [3.0, 4.0], [0.0, 0.0]]))
    assert l[0] == 0.7 and l[1] == -1.25 and np.isneginf(l[2])


def test_merge_two_equal_halves():
    """Two blocks with equal LSE: O is their average, LSE grows by ln 2."""
    o_a = np.array([[2.0, 0.0]])
    o_b = np.array([[0.0, 4.0]])
    o, l = oracle.merge(o_a, np.array([1.0]), o_b, np.array([1.0]))
    assert np.allclose(o, [[1.0, 2.0]], atol=1e-15) and abs(l[0] - (1 + math.log(2))) < 1e-15


# --------------------------------------------------------------------------- brute force

def _brute(q, k, v, ids, pos, causal, window, scale):
    b, t, hq, d = q.shape
    tk, hkv = k.shape[1], k.shape[2]
    grp = hq // hkv
    dv = v.shape[3]
    o = np.zeros((b, t, hq, dv))
    lse = np.full((b, t, hq), -np.inf)
    for bb in range(b):
        for i in range(t):
            for h in range(hq):
                g = h // grp
                scores = {}
                for j in range(tk):
                    qi, kj = int(ids[bb, i]), int(ids[bb, j])
                    pq, pk = int(pos[bb, i]), int(pos[bb, j])
                    if qi == 0 or kj == 0 or qi != kj:
                        continue
                    if causal and pk > pq:
                        continue
                    if window[0] >= 0 and pq - pk > window[0]:
                        continue
                    if window[1] >= 0 and pk - pq > window[1]:
                        continue
                    scores[j] = scale * math.fsum(float(q[bb, i, h, x]) * float(k[bb, j, g, x])
                                                  for x in range(d))
                if not scores:
                    continue
                mx = max(scores.values())
                w = {j: math.exp(s - mx) for j, s in scores.items()}
                z = math.fsum(w.values())
                for x in range(dv):
                    o[bb, i, h, x] = math.fsum(w[j] * float(v[bb, j, g, x]) for j in w) / z
                lse[bb, i, h] = mx + math.log(z)
    return o, lse


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    """P5: scalar loops with exact summation on tiny random layouts."""
    rng = np.random.default_rng(100 + seed)
    t = int(rng.integers(5, 25))
    hkv = int(rng.choice([1, 2]))
    grp = int(rng.choice([1, 2, 4]))
    d = int(rng.choice([4, 8]))
    causal = bool(rng.integers(0, 2))
    window = (int(rng.integers(-1, 8)), int(rng.integers(-1, 5)))
    ids, pos = random_layout(rng, 2, t, max_segments=3, pad_prob=0.3, pos_offset_max=4)
    q, k, v = random_qkv(2, t, t, hq := hkv * grp, hkv, d, "bf16", seed=seed)
    if seed % 2:      # V with its own head dim
        v = random_qkv(2, t, t, hq, hkv, d + 4, "bf16", seed=seed + 50)[2]
    scale = float(rng.uniform(0.2, 1.0))
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, scale=scale, causal=causal,
                              window=window)
    ob, lb = _brute(_f64(q), _f64(k), _f64(v), ids.numpy(), pos.numpy(), causal, window, scale)
    assert np.abs(o - ob).max() < 1e-12
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    f = np.isfinite(lb)
    assert np.abs(lse[f] - lb[f]).max() < 1e-12
    assert hq == q.shape[2]


def test_rows_api_equals_full():
    rng = np.random.default_rng(4)
    ids, pos = random_layout(rng, 2, 64, max_segments=3, pad_prob=0.2)
    q, k, v = random_qkv(2, 64, 64, 8, 2, 8, "bf16", seed=4)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True, window=(9, 0))
    rows = [(0, 0), (0, 13), (1, 63), (1, 30), (0, 40)]
    o2, l2 = oracle.attention_rows(q, k, v, ids, pos, ids, pos, rows, causal=True, window=(9, 0))
    for n, (b, i) in enumerate(rows):
        assert np.abs(o2[n] - o[b, i]).max() < 1e-13
        f = np.isfinite(lse[b, i])
        assert np.array_equal(f, np.isfinite(l2[n]))
        assert np.abs(l2[n][f] - lse[b, i][f]).max() < 1e-13


# --------------------------------------------------------------------------- counts

def _golden_pairs():
    out = {}
    with open(os.path.join(GOLDEN, "visible_pairs.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                cfg, total = line.split(":")[0].split()
                out[int(cfg)] = int(total)
    return out


def _closed_form_segment(n, left):
    return sum(min(p + 1, left + 1) if left >= 0 else p + 1 for p in range(n))


def test_golden_pair_totals_match_closed_forms():
    g = _golden_pairs()
    assert g[1] == _closed_form_segment(256, -1)
    assert g[2] == 2 * 4 * _closed_form_segment(768, -1)
    assert g[4] == _closed_form_segment(32768, 4096)
    assert g[5] == 2 * 4 * _closed_form_segment(12288, 8192)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_visible_pairs_of_workloads(cfg):
    """P6: the oracle's mask counts the closed-form totals of the workloads."""
    from workloads import get
    w = get(cfg)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    n = oracle.visible_pairs(ids, pos, ids, pos, w.causal, w.window)
    assert int(n.sum()) == _golden_pairs()[cfg]


def test_visible_pairs_longctx_one_slot():
    """Workload 5's rows are 4 identical slots, tiled over 2 rows; one slot's
    count times 8 is the whole total."""
    ids, pos = packed_metadata(1, 16384, 1, 12288)
    n = oracle.visible_pairs(ids, pos, ids, pos, True, (8192, 0))
    assert 8 * int(n.sum()) == _golden_pairs()[5]


# --------------------------------------------------------------------------- reorder

def _golden_maps():
    out = []
    with open(os.path.join(GOLDEN, "reorder_maps.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                head, body = line.split(":")
                kind, t, r, s = head.split()
                out.append((kind, int(t), int(r), int(s), [int(x) for x in body.split()]))
    return out


def test_reorder_maps_golden():
    """P7: hand-worked maps for both strategies."""
    maps = _golden_maps()
    assert len(maps) >= 6
    for kind, t, r, s, ref in maps:
        m = oracle.reorder_map(t, r, kind, max(s, 1))
        assert m.tolist() == ref, (kind, t, r, s)


@pytest.mark.parametrize("kind,t,r,s", [("dual_chunk", 4096, 4, 1), ("dual_chunk", 64, 8, 1),
                                        ("striped", 4096, 4, 1), ("striped", 4096, 4, 512),
                                        ("striped", 96, 3, 8)])
def test_reorder_map_is_bijection_with_inverse(kind, t, r, s):
    m = oracle.reorder_map(t, r, kind, s)
    assert sorted(m.tolist()) == list(range(t))
    inv = oracle.inverse_map(m)
    assert np.array_equal(m[inv], np.arange(t)) and np.array_equal(inv[m], np.arange(t))
    x = np.random.default_rng(0).normal(size=(2, t, 3))
    assert np.array_equal(oracle.apply_map(oracle.apply_map(x, m), inv), x)


def test_dual_chunk_balances_causal_work():
    """"Load balance": pairing early and late stripes gives every rank the
    same causal work on one unpadded causal sequence (T = 2R*c, each rank
    sees c*(c+1)/2 + ... pairs; all equal)."""
    t, r = 256, 4
    ids, pos = _contig_meta(1, t)
    m = oracle.reorder_map(t, r, "dual_chunk")
    ids_r, pos_r = oracle.apply_map(ids.numpy(), m), oracle.apply_map(pos.numpy(), m)
    n = t // r
    per_rank = [int(oracle.visible_pairs(ids_r[:, k * n:(k + 1) * n], pos_r[:, k * n:(k + 1) * n],
                                         ids_r, pos_r, True).sum()) for k in range(r)]
    assert len(set(per_rank)) == 1
    assert sum(per_rank) == t * (t + 1) // 2


# --------------------------------------------------------------------------- equivariance / ring

@pytest.mark.parametrize("kind,s", [("dual_chunk", 1), ("striped", 1), ("striped", 4)])
def test_permutation_equivariance(kind, s):
    """P9: the mask uses positions, not array indices, so attention on the
    reordered sequence, permuted back, equals attention on the original."""
    rng = np.random.default_rng(8)
    ids, pos = random_layout(rng, 2, 96, max_segments=4, pad_prob=0.2)
    q, k, v = random_qkv(2, 96, 96, 4, 2, 8, "bf16", seed=8)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True, window=(30, 0))
    m = oracle.reorder_map(96, 4, kind, s)
    ap = oracle.apply_map
    qn, kn, vn = _f64(q), _f64(k), _f64(v)
    ids_r, pos_r = ap(ids.numpy(), m), ap(pos.numpy(), m)
    o_r, l_r = oracle.attention(ap(qn, m), ap(kn, m), ap(vn, m), ids_r, pos_r, ids_r, pos_r,
                                causal=True, window=(30, 0))
    inv = oracle.inverse_map(m)
    assert np.abs(ap(o_r, inv) - o).max() < 1e-12
    lb = ap(l_r, inv)
    f = np.isfinite(lse)
    assert np.array_equal(f, np.isfinite(lb)) and np.abs(lb[f] - lse[f]).max() < 1e-12


@pytest.mark.parametrize("kind,s,window", [("dual_chunk", 1, (-1, -1)), ("dual_chunk", 1, (40, 0)),
                                           ("striped", 1, (40, 0)), ("striped", 8, (-1, -1))])
def test_ring_emulation_equals_unsplit(kind, s, window):
    """P10: reorder, per-rank ring steps with merges, inverse reorder equals
    one unsplit attention ("Ring attention": exact apart from rounding)."""
    ids, pos = packed_metadata(2, 256, 4, 48)
    q, k, v = random_qkv(2, 256, 256, 8, 2, 16, "bf16", seed=33)
    o, lse = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True, window=window)
    o2, l2 = oracle.ring_attention(q, k, v, ids, pos, ids, pos, 4, kind, s, causal=True,
                                   window=window)
    assert np.abs(o2 - o).max() < 1e-12
    f = np.isfinite(lse)
    assert np.array_equal(f, np.isfinite(l2)) and np.abs(l2[f] - lse[f]).max() < 1e-12


# --------------------------------------------------------------------------- tile classes

def _interval_classes(t, bm, bn, causal, left):
    """Classes on one unpadded segment with positions = indices, from interval
    arithmetic: the tile's query range [i0, i1] and key range [j0, j1]."""
    nq, nk = -(-t // bm), -(-t // bn)
    out = np.zeros((1, nq, nk), np.int8)
    for a in range(nq):
        i0, i1 = a * bm, min(t, (a + 1) * bm) - 1
        for c in range(nk):
            j0, j1 = c * bn, min(t, (c + 1) * bn) - 1
            lo, hi = i0 - j1, i1 - j0          # range of i - j over the tile
            ok_lo = 0 if causal else -10 ** 9  # need i - j >= ok_lo
            ok_hi = left if left >= 0 else 10 ** 9
            if hi < ok_lo or lo > ok_hi:
                out[0, a, c] = 0
            elif lo >= ok_lo and hi <= ok_hi:
                out[0, a, c] = 2
            else:
                out[0, a, c] = 1
    return out


@pytest.mark.parametrize("t,bm,bn,causal,left", [(256, 64, 64, True, -1), (300, 32, 64, True, 50),
                                                 (200, 128, 64, True, 0), (130, 16, 32, False, 40),
                                                 (517, 64, 128, True, 129)])
def test_tile_classes_interval_geometry(t, bm, bn, causal, left):
    ids, pos = _contig_meta(1, t)
    cls = oracle.classify_tiles_exact(ids, pos, ids, pos, bm, bn, causal, (left, -1))
    assert np.array_equal(cls, _interval_classes(t, bm, bn, causal, left))


def test_tile_classes_causal_triangle_counts():
    """Causal, one segment, square tiles: n diagonal tiles are partial, the
    n(n-1)/2 below are full and the n(n-1)/2 above are skipped."""
    cls = oracle.classify_tiles_exact(*_contig_meta(1, 512), *_contig_meta(1, 512), 64, 64, True)
    n = 8
    assert oracle.tile_class_counts(cls) == (n * (n - 1) // 2, n, n * (n - 1) // 2)


def test_tile_classes_padding_and_segments():
    """Padding tiles are skipped; tiles crossing into another segment are at
    most partial."""
    ids, pos = packed_metadata(1, 256, 2, 96)     # slots of 128: 96 valid + 32 pad
    cls = oracle.classify_tiles_exact(ids, pos, ids, pos, 32, 32, True)[0]
    # query tile 3 (tokens 96..127) is pure padding
    assert (cls[3] == 0).all() and (cls[:, 3] == 0).all()
    # no pair across the two slots
    assert (cls[:4, 4:] == 0).all() and (cls[4:, :4] == 0).all()
    # inside a slot: diagonal partial, below full
    assert cls[1, 1] == 1 and cls[2, 0] == 2 and cls[0, 2] == 0
