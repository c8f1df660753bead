"""GPU parity of merge, reorder and tile classification against the oracle.

Reorder maps and tile classes are integer work: they must match bit for bit.
The merge is held to the attention bar and its -inf rules exactly.
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare, to64
from workloads import get, packed_metadata, random_layout

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


# --------------------------------------------------------------------------- merge

def _partials(b, t, h, d, dtype, seed, empty_frac=0.2):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn((b, t, h, d), generator=g).to(dtype)
    lse = torch.randn((b, t, h), generator=g) * 4
    empty = torch.rand((b, t, h), generator=g) < empty_frac
    lse[empty] = -np.inf
    o[empty] = 0
    return o, lse


@pytest.mark.parametrize("da,db,dout", [(torch.float32,) * 3, (torch.bfloat16,) * 3,
                                        (torch.float32, torch.float32, torch.bfloat16),
                                        (torch.bfloat16, torch.float32, torch.float32)])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_random(da, db, dout, d):
    oa, la = _partials(2, 37, 5, d, da, 1)
    ob, lb = _partials(2, 37, 5, d, db, 2)
    # a few rows where both are empty, and huge LSE gaps
    la[0, 0, :], lb[0, 0, :] = -np.inf, -np.inf
    oa[0, 0], ob[0, 0] = 0, 0
    la[1, 3, 0], lb[1, 3, 0] = 80.0, -80.0
    o, l = bosf.attn_merge(oa.to(DEV), la.to(DEV), ob.to(DEV), lb.to(DEV), out_dtype=dout)
    ro, rl = oracle.merge(oa, la, ob, lb)
    compare(o, l, ro, rl, "bf16", "merge")
    # exactly one -inf: the other operand's row is copied unchanged
    only_a = torch.isneginf(lb) & ~torch.isneginf(la)
    if dout == da:
        assert torch.equal(o.cpu()[only_a], oa[only_a].to(dout))
        assert torch.equal(l.cpu()[only_a], la[only_a])


def test_merge_in_place_and_views():
    oa, la = _partials(2, 64, 8, 128, torch.float32, 3)
    ob, lb = _partials(2, 64, 8, 128, torch.float32, 4)
    ro, rl = oracle.merge(oa, la, ob, lb)
    oad, lad = oa.to(DEV), la.to(DEV)
    bosf.attn_merge(oad, lad, ob.to(DEV), lb.to(DEV), out=oad, lse_out=lad)
    compare(oad, lad, ro, rl, "bf16", "in place")
    # output into a batch-strided shard of a longer bf16 tensor
    big = torch.full((2, 256, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    bigl = torch.full((2, 256, 8), 3.0, device=DEV)
    bosf.attn_merge(oa.to(DEV), la.to(DEV), ob.to(DEV), lb.to(DEV), out=big[:, 64:128],
                    lse_out=bigl[:, 64:128])
    compare(big[:, 64:128], bigl[:, 64:128], ro, rl, "bf16", "view")
    assert (big[:, :64] == 3).all() and (big[:, 128:] == 3).all() and (bigl[:, 128:] == 3).all()


def test_merge_never_nan_on_large_lse():
    o = torch.ones(1, 4, 1, 64, device=DEV)
    la = torch.tensor([[[1e30], [-1e30], [88.0], [-88.0]]], device=DEV)
    lb = torch.tensor([[[1e30], [-1e30], [-88.0], [88.0]]], device=DEV)
    mo, ml = bosf.attn_merge(o, la, o, lb)
    assert torch.isfinite(mo).all() and not torch.isnan(ml).any()


# --------------------------------------------------------------------------- reorder

@pytest.mark.parametrize("t,r,kind,s", [(4096, 4, "dual_chunk", 1), (4096, 4, "striped", 1),
                                        (4096, 4, "striped", 512), (96, 3, "striped", 8),
                                        (24, 2, "dual_chunk", 1), (65536, 4, "dual_chunk", 1)])
def test_reorder_iota_bit_exact(t, r, kind, s):
    x = torch.arange(2 * t, dtype=torch.int32).reshape(2, t)
    y = bosf.reorder(x.to(DEV), r, kind, s).cpu().numpy()
    m = oracle.reorder_map(t, r, kind, s)
    assert np.array_equal(y, oracle.apply_map(x.numpy(), m))
    z = bosf.inverse_reorder(torch.from_numpy(y).to(DEV), r, kind, s).cpu().numpy()
    assert np.array_equal(z, x.numpy())


@pytest.mark.parametrize("shape,dtype", [((2, 64, 3), torch.uint8), ((2, 64, 1), torch.int16),
                                         ((2, 64, 3), torch.int16), ((1, 64, 6), torch.uint8),
                                         ((2, 64, 4, 8), torch.bfloat16),
                                         ((2, 128, 16, 128), torch.bfloat16),
                                         ((2, 64, 128, 128), torch.bfloat16),
                                         ((2, 64, 8), torch.float32)])
def test_reorder_rows_bytes(shape, dtype):
    g = torch.Generator().manual_seed(0)
    x = torch.randint(0, 120, shape, generator=g, dtype=torch.int64).to(dtype)
    t = shape[1]
    for kind, s in (("dual_chunk", 1), ("striped", 2)):
        m = oracle.reorder_map(t, 4, kind, s)
        y = bosf.reorder(x.to(DEV), 4, kind, s).cpu()
        assert torch.equal(y, x[:, torch.from_numpy(m)])
        z = bosf.inverse_reorder(y.to(DEV), 4, kind, s).cpu()
        assert torch.equal(z, x)


# --------------------------------------------------------------------------- classification

def _classify_both(q_ids, q_pos, kv_ids, kv_pos, hq, hkv, d, dtype, causal, window):
    cls, pairs = bosf.classify_tiles(q_ids.to(DEV), q_pos.to(DEV), kv_ids.to(DEV), kv_pos.to(DEV),
                                     num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                                     causal=causal, window=window)
    desc = bosf.make_desc(q_ids.shape[0], q_ids.shape[1], kv_ids.shape[1], hq, hkv, d,
                          0 if dtype == torch.bfloat16 else 1)
    bm, bn = bosf.tile_shape(desc)
    ref = oracle.classify_tiles_exact(q_ids, q_pos, kv_ids, kv_pos, bm, bn, causal, window)
    ref_pairs = oracle.visible_pairs(q_ids, q_pos, kv_ids, kv_pos, causal, window)
    return cls.cpu().numpy(), pairs.cpu().numpy(), ref, ref_pairs


@pytest.mark.parametrize("seed", range(8))
def test_classify_random_layouts(seed):
    rng = np.random.default_rng(seed)
    tq, tk = int(rng.integers(1, 700)), int(rng.integers(1, 700))
    q_ids, q_pos = random_layout(rng, 2, tq, max_segments=5, pad_prob=0.3, pos_offset_max=30)
    kv_ids, kv_pos = (q_ids, q_pos) if seed % 2 else random_layout(rng, 2, tk, 4, 0.3, 30)
    hq, hkv = [(16, 2), (4, 4), (12, 4), (8, 1)][seed % 4]
    dtype = torch.bfloat16 if seed % 3 else torch.float32
    causal = bool(seed % 2)
    window = [(-1, -1), (37, 0), (0, 0), (20, 20)][seed % 4]
    cls, pairs, ref, ref_pairs = _classify_both(q_ids, q_pos, kv_ids, kv_pos, hq, hkv, 128,
                                                dtype, causal, window)
    assert np.array_equal(cls, ref)
    assert np.array_equal(pairs, ref_pairs)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_classify_workloads(cfg):
    w = get(cfg)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cls, pairs, ref, ref_pairs = _classify_both(ids, pos, ids, pos, w.num_q_heads,
                                                w.num_kv_heads, w.head_dim, dt, w.causal, w.window)
    assert np.array_equal(cls, ref)
    assert np.array_equal(pairs, ref_pairs)


@pytest.mark.parametrize("cfg,kind", [(3, "dual_chunk"), (5, "dual_chunk"), (5, "striped")])
def test_classify_ring_steps(cfg, kind):
    """Every (rank, ring step) of the reordered workloads, batch row 0 (rows are
    identical), against the oracle on its own reordered metadata: the
    dual-chunk layout the benchmark times and the tutorial's ring layout
    (striped, stripe 1), all four ranks."""
    from concurrent.futures import ThreadPoolExecutor
    w = get(cfg)
    stripe = 1
    ids, pos = packed_metadata(1, w.seq_len, w.slots, w.valid_per_slot)
    m = oracle.reorder_map(w.seq_len, w.cp_size, kind, stripe)
    ids_o, pos_o = oracle.apply_map(ids.numpy(), m), oracle.apply_map(pos.numpy(), m)
    ids_g = bosf.reorder(ids.to(DEV), w.cp_size, kind, stripe)
    pos_g = bosf.reorder(pos.to(DEV), w.cp_size, kind, stripe)
    assert np.array_equal(ids_g.cpu().numpy(), ids_o)
    n = w.seq_len // w.cp_size
    desc = bosf.make_desc(1, n, n, w.num_q_heads, w.num_kv_heads, w.head_dim)
    bm, bn = bosf.tile_shape(desc)
    steps = [(r, s) for r in range(w.cp_size) for s in range(w.cp_size)]
    got, total = {}, 0
    for r, s in steps:
        rq = slice(r * n, (r + 1) * n)
        c = (r - s) % w.cp_size
        rk = slice(c * n, (c + 1) * n)
        cls, pairs = bosf.classify_tiles(ids_g[:, rq], pos_g[:, rq], ids_g[:, rk], pos_g[:, rk],
                                         num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                                         head_dim=w.head_dim, causal=w.causal, window=w.window)
        got[(r, s)] = cls.cpu().numpy()
        total += int(pairs.cpu()[0])

    def exact(rs):
        r, s = rs
        c = (r - s) % w.cp_size
        rq, rk = slice(r * n, (r + 1) * n), slice(c * n, (c + 1) * n)
        return oracle.classify_tiles_exact(ids_o[:, rq], pos_o[:, rq], ids_o[:, rk], pos_o[:, rk],
                                           bm, bn, w.causal, w.window)

    with ThreadPoolExecutor(8) as ex:
        refs = dict(zip(steps, ex.map(exact, steps)))
    for rs in steps:
        assert np.array_equal(got[rs], refs[rs]), rs
    # the ring covers every visible pair of one batch row exactly once
    want = int(oracle.visible_pairs(ids, pos, ids, pos, w.causal, w.window)[0])
    assert total == want
    if cfg == 5:
        assert total == 536936448 // 2
