"""GPU test of the forward entry point that allocates nothing
(``ra_attn_fwd_noalloc``): its outputs equal ``ra_attn_fwd``'s bit for bit
and meet the oracle's bar, on two calls in a row (the second smaller than the
first, so stale scratch contents from the first call must not leak into it),
on the fp32 path, on the largest workload that fits the scratch, and a call
that needs more scratch than the library holds is refused before any launch.
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare
from workloads import get, packed_metadata, random_layout, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _both(q, k, v, qi, qp, ki, kp, **kw):
    ref = bosf.attn_fwd(q, k, v, qi, qp, ki, kp, **kw)
    out = torch.full_like(ref[0], 5.0)
    lse = torch.full_like(ref[1], 5.0)
    got = bosf.attn_fwd_noalloc(q, k, v, qi, qp, ki, kp, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_two_calls_second_smaller():
    big = dict(b=2, t=1024, hq=16, hkv=2, d=128)
    ids, pos = packed_metadata(2, 1024, 2, 400)
    q, k, v = random_qkv(2, 1024, 1024, 16, 2, 128, "bf16", seed=41)
    kw = dict(causal=True, window=(300, 0))
    dev = [t.to(DEV) for t in (q, k, v, ids, pos)]
    (ro, rl), (go, gl) = _both(*dev[:3], dev[3], dev[4], dev[3], dev[4], **kw)
    assert torch.equal(go, ro) and torch.equal(gl, rl)
    oo, ol = oracle.attention(q, k, v, ids, pos, ids, pos, **kw)
    compare(go, gl, oo, ol, "bf16", f"noalloc first call {big}")
    # second call, smaller, other layout and head dim: only what this call wrote is read
    rng = np.random.default_rng(42)
    qi, qp = random_layout(rng, 1, 300, max_segments=4, pad_prob=0.3, pos_offset_max=3)
    ki, kp = random_layout(rng, 1, 200, max_segments=3, pad_prob=0.3, pos_offset_max=30)
    q2, k2, v2 = random_qkv(1, 300, 200, 8, 1, 64, "bf16", seed=43)
    kw2 = dict(causal=False, window=(40, 40))
    dev2 = [t.to(DEV) for t in (q2, k2, v2, qi, qp, ki, kp)]
    (ro2, rl2), (go2, gl2) = _both(*dev2, **kw2)
    assert torch.equal(go2, ro2) and torch.equal(gl2, rl2)
    oo2, ol2 = oracle.attention(q2, k2, v2, qi, qp, ki, kp, **kw2)
    compare(go2, gl2, oo2, ol2, "bf16", "noalloc second, smaller call")


def test_noalloc_fp32_and_largest_fitting_workload():
    w = get(1)
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    q, k, v = random_qkv(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                         w.head_dim, "f32", seed=w.seed)
    dev = [t.to(DEV) for t in (q, k, v, ids, pos)]
    (ro, rl), (go, gl) = _both(*dev[:3], dev[3], dev[4], dev[3], dev[4], causal=True)
    assert torch.equal(go, ro) and torch.equal(gl, rl)
    oo, ol = oracle.attention(q, k, v, ids, pos, ids, pos, causal=True)
    compare(go, gl, oo, ol, "f32", "noalloc fp32")
    # the sliding-window workload (one call over 32768 tokens) fits the scratch
    w = get(4)
    desc = bosf.make_desc(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, window=w.window)
    assert bosf.workspace_size(desc) <= bosf.NOALLOC_SCRATCH_BYTES
    g = torch.Generator(device=DEV).manual_seed(w.seed)
    shp = (w.batch, w.seq_len)
    q = torch.randn(shp + (w.num_q_heads, w.head_dim), generator=g, device=DEV).bfloat16()
    k = torch.randn(shp + (w.num_kv_heads, w.head_dim), generator=g, device=DEV).bfloat16()
    v = torch.randn(shp + (w.num_kv_heads, w.head_dim), generator=g, device=DEV).bfloat16()
    ids, pos = (t.to(DEV) for t in packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot))
    (ro, rl), (go, gl) = _both(q, k, v, ids, pos, ids, pos, causal=True, window=w.window)
    assert torch.equal(go, ro) and torch.equal(gl, rl)


def test_noalloc_refuses_more_than_its_scratch():
    ids = torch.ones((2, 65536), dtype=torch.int32, device=DEV)
    pos = torch.arange(65536, dtype=torch.int32, device=DEV).repeat(2, 1)
    q = torch.zeros((2, 64, 8, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((2, 65536, 8, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full((2, 64, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((2, 64, 8), 3.0, device=DEV)
    with pytest.raises(bosf.RingAttnError, match="RA_ERR_WORKSPACE"):
        bosf.attn_fwd_noalloc(q, k, k, ids[:, :64], pos[:, :64], ids, pos, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out == 3.0).all() and (lse == 3.0).all()
