"""GPU parity at the largest lengths the library accepts.

The forward takes up to 32768 key tiles of 64 tokens (2^21 keys) per call, and
the backward up to 32768 query tiles of 32 tokens (2^20 queries).  Both limits
are exercised at exactly that size, with few heads so the oracle stays cheap,
and the next size up must be refused before any launch.
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare, compare_grads

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _randn(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


def test_forward_at_the_key_length_limit():
    """64 queries against 2^21 keys of one segment: the last 64 positions, each
    seeing every earlier key (causal), checked on sampled rows; one key more is
    refused."""
    tk, tq, d = 64 * 32768, 64, 64
    q = _randn((1, tq, 1, d), 1)
    k = _randn((1, tk, 1, d), 2)
    v = _randn((1, tk, 1, d), 3)
    kid = torch.ones((1, tk), dtype=torch.int32, device=DEV)
    kpos = torch.arange(tk, dtype=torch.int32, device=DEV)[None]
    qid = torch.ones((1, tq), dtype=torch.int32, device=DEV)
    qpos = kpos[:, tk - tq:].contiguous()
    o, lse = bosf.attn_fwd(q, k, v, qid, qpos, kid, kpos)
    torch.cuda.synchronize()
    rows = [(0, 0), (0, 17), (0, tq - 1)]
    ro, rl = oracle.attention_rows(q, k.cpu(), v.cpu(), qid.cpu(), qpos.cpu(), kid.cpu(),
                                   kpos.cpu(), rows)
    bi = torch.tensor([r[0] for r in rows])
    ti = torch.tensor([r[1] for r in rows])
    compare(o[bi, ti], lse[bi, ti], ro, rl, "bf16", "2^21 keys")
    k1 = torch.zeros((1, tk + 1, 1, d), dtype=torch.bfloat16, device=DEV)
    ids1 = torch.ones((1, tk + 1), dtype=torch.int32, device=DEV)
    with pytest.raises(bosf.RingAttnError, match="RA_ERR_UNSUPPORTED"):
        bosf.attn_fwd(q, k1, k1, qid, qpos, ids1, ids1)


def test_backward_at_the_query_length_limit():
    """2^20 queries in one segment against 64 keys (non-causal): dQ on sampled
    rows; dK and dV of every key (each seen by all 2^20 queries) against the
    oracle; one query more is refused."""
    tq, tk, d = 32 * 32768, 64, 64
    q = _randn((1, tq, 1, d), 4)
    k = _randn((1, tk, 1, d), 5)
    v = _randn((1, tk, 1, d), 6)
    do = _randn((1, tq, 1, d), 7)
    qid = torch.ones((1, tq), dtype=torch.int32, device=DEV)
    qpos = torch.arange(tq, dtype=torch.int32, device=DEV)[None]
    kid = torch.ones((1, tk), dtype=torch.int32, device=DEV)
    kpos = torch.arange(tk, dtype=torch.int32, device=DEV)[None]
    kw = dict(causal=False)
    o, lse = bosf.attn_fwd(q, k, v, qid, qpos, kid, kpos, **kw)
    dq, dk, dv = bosf.attn_bwd(q, k, v, qid, qpos, kid, kpos, o, lse, do, **kw)
    torch.cuda.synchronize()
    host = [t.cpu() for t in (q, k, v, do, qid, qpos, kid, kpos)]
    rows = [(0, 0), (0, 12345), (0, tq - 1)]
    rq = oracle.backward_query_rows(*host, rows, **kw)
    compare_grads(dq[0, [r[1] for r in rows]], rq, "dq at 2^20 queries")
    keys = [(0, j) for j in (0, 31, 63)]
    rk, rv = oracle.backward_key_rows(*host, keys, **kw)
    compare_grads(dk[0, [j for _, j in keys]], rk, "dk at 2^20 queries")
    compare_grads(dv[0, [j for _, j in keys]], rv, "dv at 2^20 queries")
    q1 = torch.zeros((1, tq + 1, 1, d), dtype=torch.bfloat16, device=DEV)
    ids1 = torch.ones((1, tq + 1), dtype=torch.int32, device=DEV)
    with pytest.raises(bosf.RingAttnError, match="RA_ERR_UNSUPPORTED"):
        bosf.attn_bwd(q1, k, v, ids1, ids1, kid, kpos, q1, torch.zeros((1, tq + 1, 1), device=DEV),
                      q1, **kw)
