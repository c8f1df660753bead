"""GPU parity of the bf16 forward with MLA head dimensions (Q/K head dim 192,
V and O head dim 128) against the fp64 oracle.

Small cases cover every workgroup shape (GQA groups 1, 2, 3, 8, 16), windows,
cross-attention, fp32 output, the accumulating forward and the all-gather
driver; the MLA workload (2 x 8192 tokens, 128 heads) is checked at full size
on sampled rows and, with Q = 0, on every row through its closed form
(LSE = ln n, O = the mean of the visible V rows).
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
import oracle
from _parity import compare
from _workload_io import closed_form_counts, device_inputs, sample_rows
from workloads import get, random_layout, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"
D, DV = 192, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def _dev(*ts):
    return [t.to(DEV) for t in ts]


# (B, Tq, Tk, Hq, Hkv, causal, window, self_attention)
SMALL = [
    (1, 1, 1, 1, 1, True, (-1, -1), True),
    (2, 257, 257, 16, 2, True, (-1, -1), True),
    (1, 300, 300, 8, 8, True, (40, 0), True),
    (2, 200, 200, 32, 2, True, (0, 0), True),
    (1, 250, 250, 8, 4, False, (17, 9), True),
    (2, 129, 129, 3, 1, True, (-1, 5), True),
    (2, 300, 517, 16, 1, True, (-1, -1), False),
    (1, 517, 300, 4, 4, False, (50, 50), False),
]


def _cid(c):
    b, tq, tk, hq, hkv, causal, w, self_ = c
    return f"B{b}_Tq{tq}_Tk{tk}_H{hq}-{hkv}_{'c' if causal else 'nc'}_w{w[0]}.{w[1]}_{'self' if self_ else 'cross'}"


def _small(case, seed):
    b, tq, tk, hq, hkv, causal, window, self_ = case
    rng = np.random.default_rng(seed)
    qi, qp = random_layout(rng, b, tq, max_segments=4, pad_prob=0.25, pos_offset_max=3)
    if self_:
        ki, kp = qi, qp
    else:
        ki, kp = random_layout(rng, b, tk, max_segments=3, pad_prob=0.25, pos_offset_max=40)
    q, k, v = random_qkv(b, tq, tk, hq, hkv, D, "bf16", seed=seed, dv=DV)
    return q, k, v, qi, qp, ki, kp


@pytest.mark.parametrize("case", SMALL, ids=[_cid(c) for c in SMALL])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_mla_small(case, out):
    causal, window = case[5], case[6]
    q, k, v, qi, qp, ki, kp = _small(case, case[1] * 3 + case[2])
    o, lse = bosf.attn_fwd(*_dev(q, k, v, qi, qp, ki, kp), causal=causal, window=window,
                           out_dtype=torch.float32 if out == "f32" else None)
    torch.cuda.synchronize()
    assert o.shape == (case[0], case[1], case[3], DV)
    ro, rl = oracle.attention(q, k, v, qi, qp, ki, kp, causal=causal, window=window)
    compare(o, lse, ro, rl, "bf16", f"MLA {_cid(case)} out {out}")


def test_mla_accumulate_and_allgather():
    """Folding two key blocks with attn_fwd_accumulate equals one call over both;
    the all-gather driver on MLA shapes matches the oracle."""
    b, t, hq, hkv = 2, 512, 16, 2
    q, k, v = random_qkv(b, t, t, hq, hkv, D, "bf16", seed=9, dv=DV)
    ids = torch.ones((b, t), dtype=torch.int32)
    pos = torch.arange(t, dtype=torch.int32)[None].repeat(b, 1)
    qd, kd, vd, idd, pod = _dev(q, k, v, ids, pos)
    h = t // 2
    po, pl = bosf.attn_fwd(qd, kd[:, :h], vd[:, :h], idd, pod, idd[:, :h], pod[:, :h],
                           out_dtype=torch.float32)
    bosf.attn_fwd_accumulate(qd, kd[:, h:], vd[:, h:], idd, pod, idd[:, h:], pod[:, h:], po, pl)
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos)
    compare(po, pl, ro, rl, "bf16", "MLA accumulate")
    o, lse = bosf.allgather_forward(qd, kd, vd, idd, pod, 4, "striped", 64, window=(200, 0))
    ro, rl = oracle.attention(q, k, v, ids, pos, ids, pos, window=(200, 0))
    compare(o, lse, ro, rl, "bf16", "MLA all-gather")


def test_mla_workload_full_size_sampled():
    w = get(6)
    q, k, v, ids, pos = device_inputs(w)
    o, lse = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(66)
    rows = sample_rows(w, rng, [0, 1, 63, 64, 255, 256, 4095, 4096, w.seq_len - 1], n_random=8)
    ro, rl = oracle.attention_rows(q, k.cpu(), v.cpu(), ids.cpu(), pos.cpu(), ids.cpu(),
                                   pos.cpu(), rows, causal=w.causal, window=w.window)
    bi = torch.tensor([r[0] for r in rows])
    ti = torch.tensor([r[1] for r in rows])
    e = compare(o[bi, ti], lse[bi, ti], ro, rl, "bf16", "MLA workload")
    print(f"MLA workload: {len(rows)} rows x {w.num_q_heads} heads: max|dO|={e[0]:.2e} "
          f"max|dLSE|={e[1]:.2e}")


def test_mla_workload_zero_queries_every_row():
    """Q = 0: every visible score is 0, so LSE = ln n and O is the mean of the
    visible V rows (causal single segment: the prefix mean), on every row."""
    w = get(6)
    q, k, v, ids, pos = device_inputs(w, zero_q=True)
    o, lse = bosf.attn_fwd(q, k, v, ids, pos, ids, pos, causal=w.causal, window=w.window)
    nvis = closed_form_counts(w, pos, ids)
    err_l = (lse.double() - torch.log(nvis)[:, :, None]).abs().max().item()
    assert err_l <= 1e-5, err_l
    vm = v.double().cumsum(1) / nvis[:, :, None, None]               # [B, T, Hkv, Dv]
    err_o = (o.double() - vm).abs().max().item()                     # Hq == Hkv here
    print(f"MLA Q=0: max|dLSE|={err_l:.2e} max|dO|={err_o:.2e}")
    assert err_o <= 2e-2, err_o


# ----------------------------------------------------------------------------- backward

def _mla_bwd(q, k, v, qi, qp, ki, kp, do, causal, window, grad_dtype=torch.float32):
    o, lse = bosf.attn_fwd(q, k, v, qi, qp, ki, kp, causal=causal, window=window)
    return bosf.attn_bwd(q, k, v, qi, qp, ki, kp, o, lse, do, causal=causal, window=window,
                         grad_dtype=grad_dtype)


@pytest.mark.parametrize("case", SMALL, ids=[_cid(c) for c in SMALL])
def test_mla_backward_small(case):
    """dQ (192 wide), dK (192) and dV (128) of the MLA head dims against the
    fp64 backward oracle, element by element; rows and keys that no visible
    pair reaches must be exactly 0."""
    from test_gpu_bwd import _unreached
    from _parity import compare_grads
    causal, window = case[5], case[6]
    q, k, v, qi, qp, ki, kp = _small(case, case[1] * 7 + case[2])
    do = random_qkv(case[0], case[1], 1, case[3], 1, DV, "bf16", seed=case[1] + 91)[0]
    dq, dk, dv = _mla_bwd(*_dev(q, k, v, qi, qp, ki, kp, do), causal, window)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    rq, rk, rv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, causal=causal, window=window)
    zq, zk = _unreached(qi.numpy(), qp.numpy(), ki.numpy(), kp.numpy(), causal, window)
    what = f"MLA {_cid(case)}"
    compare_grads(dq, rq, what + " dq", exact_zero=np.broadcast_to(zq[:, :, None, None], rq.shape))
    compare_grads(dk, rk, what + " dk", exact_zero=np.broadcast_to(zk[:, :, None, None], rk.shape))
    compare_grads(dv, rv, what + " dv", exact_zero=np.broadcast_to(zk[:, :, None, None], rv.shape))


def test_mla_backward_bf16_gradients_and_determinism():
    from _parity import compare_grads
    case = SMALL[2]
    causal, window = case[5], case[6]
    q, k, v, qi, qp, ki, kp = _small(case, 5)
    do = random_qkv(case[0], case[1], 1, case[3], 1, DV, "bf16", seed=6)[0]
    args = _dev(q, k, v, qi, qp, ki, kp, do)
    g1 = _mla_bwd(*args, causal, window, grad_dtype=torch.bfloat16)
    g2 = _mla_bwd(*args, causal, window, grad_dtype=torch.bfloat16)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    refs = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, causal=causal, window=window)
    for got, ref, n in zip(g1, refs, ("dq", "dk", "dv")):
        assert got.dtype == torch.bfloat16
        compare_grads(got, ref, f"MLA bf16 {n}")


def test_mla_backward_workload_sampled_and_identities():
    """The MLA workload (2 x 8192 tokens, 128 heads, causal) at full size:
    sampled query rows and keys against the oracle, and per segment the keys'
    dK summing to 0 and their dV to the summed dO."""
    from test_gpu_bwd import _device_do, _sampled_check, _segment_identities
    w = get(6)
    q, k, v, ids, pos = device_inputs(w)
    do = _device_do(w, q.shape[:3] + (w.dv,))
    dq, dk, dv = _mla_bwd(q, k, v, ids, pos, ids, pos, do, w.causal, w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(61)
    rows = sorted({(int(rng.integers(0, w.batch)), int(t)) for t in rng.integers(0, w.seq_len, 6)} |
                  {(0, 0), (1, w.seq_len - 1), (0, 4095)})
    keys = sorted({(b, t) for b in range(w.batch) for t in (w.seq_len - 1, w.seq_len - 2,
                                                           w.seq_len - 40)})
    e = _sampled_check(w, q, k, v, ids, pos, ids, pos, do, dq, dk, dv, rows, keys, "MLA")
    ident = _segment_identities(dk, dv, do, ids, ids, w.group, "MLA")
    print("MLA backward sampled:", e, "identities:", ident)
