"""GPU parity of the ring step replayed from a captured HIP graph (RingGraph).

Every replay must equal, bit for bit, the eager ring driver on the same
inputs, and the eager result stays tied to the oracle.  Each graph is
replayed several times with new Q/K/V, with the program's own eager work
(other library calls, host synchronisation) between the replays, and every
replay is checked, since a wrong graph node can show only on replays after
the first.
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare
from _workload_io import device_inputs
from workloads import get, packed_metadata, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _fresh(shape_like, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return [torch.randn(t.shape, generator=g, device=DEV).to(t.dtype) for t in shape_like]


def _replays(graph, q, k, v, ids, pos, cp, kind, stripe, plan, kw, rounds=3, seed=100):
    """Replay with new inputs each round; compare with the eager driver."""
    for i in range(rounds):
        qn, kn, vn = _fresh((q, k, v), seed + i)
        o_g, l_g = graph.replay(qn, kn, vn)
        o_g, l_g = o_g.clone(), l_g.clone()
        # the program's own eager work between replays
        o_e, l_e = bosf.ring_forward(qn, kn, vn, ids, pos, cp, kind, stripe, plan=plan, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {i}: O differs from the eager ring"
        assert torch.equal(l_g, l_e), f"replay {i}: LSE differs from the eager ring"
    return qn, kn, vn, o_g, l_g


@pytest.mark.parametrize("kind,halves", [("dual_chunk", True), ("dual_chunk", False),
                                         ("striped", False)])
def test_ring_graph_small_layouts(kind, halves):
    b, t, hq, hkv, d, cp = 2, 2048, 8, 2, 128, 4
    ids, pos = packed_metadata(b, t, 4, 450)
    q, k, v = (x.to(DEV) for x in random_qkv(b, t, t, hq, hkv, d, "bf16", seed=41))
    ids, pos = ids.to(DEV), pos.to(DEV)
    kw = dict(causal=True, window=(300, 0))
    plan = bosf.ring_plan(ids, pos, cp, kind, 1, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                          dtype=q.dtype, halves=halves, **kw)
    graph = bosf.RingGraph(q, k, v, ids, pos, cp, kind, 1, plan=plan, **kw)
    o0, l0 = bosf.ring_forward(q, k, v, ids, pos, cp, kind, 1, plan=plan, **kw)
    o1, l1 = graph.replay()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    qn, kn, vn, o_g, l_g = _replays(graph, q, k, v, ids, pos, cp, kind, 1, plan, kw)
    ro, rl = oracle.attention(qn.cpu(), kn.cpu(), vn.cpu(), ids.cpu(), pos.cpu(), ids.cpu(),
                              pos.cpu(), **kw)
    compare(o_g, l_g, ro, rl, "bf16", f"graph replay {kind} halves={halves}")


def test_ring_graph_sharded_packed_workload():
    """The sharded packed workload (4 shards x 4 ring steps) at full size."""
    w = get(3)
    q, k, v, ids, pos = device_inputs(w)
    kw = dict(causal=w.causal, window=w.window)
    plan = bosf.ring_plan(ids, pos, w.cp_size, w.reorder, w.stripe, num_q_heads=w.num_q_heads,
                          num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, dtype=q.dtype,
                          halves=True, **kw)
    graph = bosf.RingGraph(q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe, plan=plan, **kw)
    qn, kn, vn, o_g, l_g = _replays(graph, q, k, v, ids, pos, w.cp_size, w.reorder, w.stripe,
                                    plan, kw, rounds=3, seed=200)
    rng = np.random.default_rng(5)
    rows = [(int(bb), int(i)) for bb in range(w.batch)
            for i in rng.choice(w.seq_len, 48, replace=False)]
    ro, rl = oracle.attention_rows(qn.cpu(), kn.cpu(), vn.cpu(), ids.cpu(), pos.cpu(), ids.cpu(),
                                   pos.cpu(), rows, **kw)
    bi = torch.tensor([r[0] for r in rows], device=DEV)
    ti = torch.tensor([r[1] for r in rows], device=DEV)
    compare(o_g[bi, ti], l_g[bi, ti], ro, rl, "bf16", "graph replay, sharded packed workload")


def test_ring_graph_replay_checks_inputs():
    b, t, hq, hkv, d, cp = 1, 1024, 4, 4, 64, 2
    ids, pos = packed_metadata(b, t, 2, 400)
    q, k, v = (x.to(DEV) for x in random_qkv(b, t, t, hq, hkv, d, "bf16", seed=43))
    ids, pos = ids.to(DEV), pos.to(DEV)
    plan = bosf.ring_plan(ids, pos, cp, "dual_chunk", 1, num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=d, dtype=q.dtype, causal=True)
    graph = bosf.RingGraph(q, k, v, ids, pos, cp, "dual_chunk", 1, plan=plan, causal=True)
    with pytest.raises(ValueError):
        graph.replay(q[:, : t // 2])
    with pytest.raises(ValueError):
        graph.replay(k=k.float())
    with pytest.raises(TypeError):
        bosf.RingGraph(q, k, v, ids, pos, cp, "dual_chunk", 1, plan=plan.counts, causal=True)
    # the graph still replays correctly after the refused calls
    o, l = graph.replay(q, k, v)
    o_e, l_e = bosf.ring_forward(q, k, v, ids, pos, cp, "dual_chunk", 1, plan=plan, causal=True)
    assert torch.equal(o, o_e) and torch.equal(l, l_e)
