"""GPU tests of the tensor layouts the library reads and writes through token
strides: packed K/V (THD_T2HD), packed Q/K/V, and sequence-major (SBHD)
tensors, in the forward, the accumulating forward and the backward.

The kernels do the same arithmetic in the same order whatever the strides, so
every layout must give results bit-identical to the same call on contiguous
copies; one case per path is also held to the oracle.
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare, compare_grads
from workloads import random_layout, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _inputs(b, t, hq, hkv, d, dtype="bf16", seed=0):
    rng = np.random.default_rng(seed)
    ids, pos = random_layout(rng, b, t, max_segments=3, pad_prob=0.2, pos_offset_max=5)
    q, k, v = random_qkv(b, t, t, hq, hkv, d, dtype, seed=seed)
    return q.to(DEV), k.to(DEV), v.to(DEV), ids.to(DEV), pos.to(DEV), (q, k, v, ids, pos)


def _packed_qkv(q, k, v):
    """Views q, k, v into one [B, T, Hq + 2 Hkv, D] buffer (packed Q/K/V)."""
    hq, hkv = q.shape[2], k.shape[2]
    buf = torch.cat([q, k, v], dim=2).contiguous()
    return buf[:, :, :hq], buf[:, :, hq:hq + hkv], buf[:, :, hq + hkv:], buf


def _packed_kv(k, v):
    """Views k, v into one [B, T, 2, Hkv, D] buffer (T2HD)."""
    buf = torch.stack([k, v], dim=2).contiguous()
    return buf[:, :, 0], buf[:, :, 1], buf


def _seq_major(x):
    """The same values held sequence-major: storage [T, B, H, D], viewed as [B, T, H, D]."""
    return x.transpose(0, 1).contiguous().transpose(0, 1)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("layout", ["packed_qkv", "packed_kv", "seq_major"])
def test_forward_layouts_bit_identical(layout, dtype, d):
    b, t, hq, hkv = 2, 333, 8, 2
    q, k, v, ids, pos, host = _inputs(b, t, hq, hkv, d, dtype, seed=7 + d)
    kw = dict(causal=True, window=(100, 0))
    o_ref, l_ref = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, **kw)
    out = None
    if layout == "packed_qkv":
        qv, kv_, vv, _ = _packed_qkv(q, k, v)
    elif layout == "packed_kv":
        qv = q
        kv_, vv, _ = _packed_kv(k, v)
    else:
        qv, kv_, vv = _seq_major(q), _seq_major(k), _seq_major(v)
        out = _seq_major(torch.zeros_like(q))
    o, lse = bosf.attn_fwd(qv, kv_, vv, ids, pos, ids, pos, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), layout
    if layout == "seq_major":
        assert o.data_ptr() == out.data_ptr() and o.stride(1) == b * hq * d
    if layout == "packed_qkv" and d == 128:
        ro, rl = oracle.attention(*host[:3], host[3], host[4], host[3], host[4], **kw)
        compare(o, lse, ro, rl, dtype, f"{layout} {dtype} D{d}")


def test_accumulate_seq_major_partial():
    """attn_fwd_accumulate in place on a sequence-major fp32 partial equals the
    same fold on a contiguous partial."""
    b, t, hq, hkv, d = 2, 260, 16, 2, 128
    q, k, v, ids, pos, _ = _inputs(b, t, hq, hkv, d, seed=3)
    k2, v2 = random_qkv(b, t, t, hq, hkv, d, "bf16", seed=4, device=DEV)[1:]
    kw = dict(causal=False, window=(-1, -1))
    pc, lc = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, out_dtype=torch.float32, **kw)
    ps = _seq_major(torch.zeros_like(pc))
    ls = torch.empty_like(lc)
    bosf.attn_fwd(_seq_major(q), k, v, ids, pos, ids, pos, out=ps, lse=ls,
                  out_dtype=torch.float32, **kw)
    bosf.attn_fwd_accumulate(q, k2, v2, ids, pos, ids, pos, pc, lc, **kw)
    bosf.attn_fwd_accumulate(_seq_major(q), k2, v2, ids, pos, ids, pos, ps, ls, **kw)
    torch.cuda.synchronize()
    assert torch.equal(ps, pc) and torch.equal(ls, lc)


@pytest.mark.parametrize("layout", ["packed_qkv", "packed_kv", "seq_major"])
def test_backward_layouts_bit_identical(layout):
    """Gradients written into the matching packed or sequence-major layout equal
    the contiguous call bit for bit; one layout is also held to the oracle."""
    b, t, hq, hkv, d = 2, 300, 8, 2, 128
    q, k, v, ids, pos, host = _inputs(b, t, hq, hkv, d, seed=11)
    do = random_qkv(b, t, 1, hq, 1, d, "bf16", seed=12, device=DEV)[0]
    kw = dict(causal=True, window=(64, 0))
    o, lse = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, **kw)
    gq, gk, gv = bosf.attn_bwd(q, k, v, ids, pos, ids, pos, o, lse, do, **kw)
    if layout == "packed_qkv":
        qv, kv_, vv, _ = _packed_qkv(q, k, v)
        gbuf = torch.full((b, t, hq + 2 * hkv, d), 5.0, device=DEV)
        dq, dk, dv = gbuf[:, :, :hq], gbuf[:, :, hq:hq + hkv], gbuf[:, :, hq + hkv:]
        ov, dov = o, do
    elif layout == "packed_kv":
        qv = q
        kv_, vv, _ = _packed_kv(k, v)
        gbuf = torch.full((b, t, 2, hkv, d), 5.0, device=DEV)
        dq, dk, dv = torch.empty_like(q, dtype=torch.float32), gbuf[:, :, 0], gbuf[:, :, 1]
        ov, dov = o, do
    else:
        qv, kv_, vv, ov, dov = (_seq_major(x) for x in (q, k, v, o, do))
        dq = _seq_major(torch.zeros_like(q, dtype=torch.float32))
        dk = _seq_major(torch.zeros_like(k, dtype=torch.float32))
        dv = _seq_major(torch.zeros_like(k, dtype=torch.float32))
    r = bosf.attn_bwd(qv, kv_, vv, ids, pos, ids, pos, ov, lse, dov, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    assert all(x.data_ptr() == y.data_ptr() for x, y in zip(r, (dq, dk, dv)))
    assert torch.equal(dq, gq) and torch.equal(dk, gk) and torch.equal(dv, gv), layout
    if layout == "packed_kv":
        rq, rk, rv = oracle.attention_backward(*host[:3], do.cpu(), host[3], host[4], host[3],
                                               host[4], **kw)
        compare_grads(dk, rk, "packed kv dk")
        compare_grads(dv, rv, "packed kv dv")
        compare_grads(dq, rq, "packed kv dq")
