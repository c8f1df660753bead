"""Host checks of the test infrastructure the full-size GPU tests rely on
(no GPU): the stratified row sample covers every query tile of every launch,
and the oracle's process pool returns exactly what its serial row functions
return."""

import numpy as np
import pytest

import oracle
from _workload_io import stratified_rows, tiles_covered
from workloads import get, packed_metadata, random_layout, random_qkv


@pytest.mark.parametrize("cfg", [4, 5])
def test_stratified_rows_cover_every_tile_of_every_layout(cfg):
    w = get(cfg)
    rows = stratified_rows(w, np.random.default_rng(cfg))
    assert len(rows) == len(set(rows)) == w.batch * w.seq_len // 32
    n_tiles = w.batch * w.seq_len // 32
    assert len(tiles_covered(rows, np.arange(w.seq_len))) == n_tiles
    for kind in ("dual_chunk", "striped"):
        m = oracle.reorder_map(w.seq_len, 4, kind, 1)
        assert len(tiles_covered(rows, m)) == n_tiles, kind


def test_pool_rows_equal_serial_rows():
    """The pool adds no arithmetic: pooled rows are bit-identical to the serial
    row functions and agree with the whole-tensor oracle."""
    rng = np.random.default_rng(5)
    ids, pos = random_layout(rng, 2, 700, max_segments=5, pad_prob=0.2, pos_offset_max=4)
    q, k, v = random_qkv(2, 700, 700, 8, 2, 64, "bf16", seed=6)
    do = random_qkv(2, 700, 1, 8, 1, 64, "bf16", seed=7)[0]
    rows = [(b, i) for b in range(2) for i in range(0, 700, 9)]
    kw = dict(causal=True, window=(90, 0))
    o1, l1 = oracle.attention_rows(q, k, v, ids, pos, ids, pos, rows, workers=1, **kw)
    o2, l2 = oracle.attention_rows(q, k, v, ids, pos, ids, pos, rows, workers=2, **kw)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, **kw)
    bi, ti = [r[0] for r in rows], [r[1] for r in rows]
    assert np.allclose(o1, ro[bi, ti], rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(l1), np.isneginf(rl[bi, ti]))
    live = ~np.isneginf(l1)
    assert np.allclose(l1[live], rl[bi, ti][live], rtol=0, atol=1e-12)
    d1 = oracle.backward_query_rows(q, k, v, do, ids, pos, ids, pos, rows, workers=1, **kw)
    d2 = oracle.backward_query_rows(q, k, v, do, ids, pos, ids, pos, rows, workers=2, **kw)
    assert np.array_equal(d1, d2)
    rq = oracle.attention_backward(q, k, v, do, ids, pos, ids, pos, **kw)[0]
    assert np.allclose(d1, rq[bi, ti], rtol=0, atol=1e-10)


def test_pool_worker_count_and_cpu_model():
    from oracle.pool import cpu_model, pool_workers
    assert 1 <= pool_workers()
    assert isinstance(cpu_model(), str) and cpu_model()
