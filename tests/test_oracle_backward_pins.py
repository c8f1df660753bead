"""Pins of the fp64 backward oracle against sources other than itself.

* torch autograd (fp64, CPU) through the plain masked attention written with
  torch ops: an independent differentiation of the same definition;
* central finite differences of L = <O, dO> (forward from the forward
  oracle) along random directions in q, k and v;
* closed forms: uniform V gives dQ = dK = 0 and dV = P^T dO; a single visible
  key per row (window (0, 0)) gives dQ = dK = 0 and dV_j = sum of the dO rows
  that see key j;
* invariants: keys' gradients sum to zero per head group (softmax is
  unchanged by a common shift of the keys); dO = 0 gives zero gradients;
  rows without a visible key contribute nothing;
* the sampled-row and sampled-key variants equal the full computation.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import random_layout

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(seed, b=2, tq=37, tk=45, hq=4, hkv=2, d=16, self_attn=False):
    rng = np.random.default_rng(seed)
    q_ids, q_pos = random_layout(rng, b, tq, max_segments=3, pad_prob=0.2)
    if self_attn:
        k_ids, k_pos = q_ids, q_pos
        tk = tq
    else:
        k_ids, k_pos = random_layout(rng, b, tk, max_segments=3, pad_prob=0.2, pos_offset_max=9)
    q = rng.standard_normal((b, tq, hq, d))
    k = rng.standard_normal((b, tk, hkv, d))
    v = rng.standard_normal((b, tk, hkv, d))
    do = rng.standard_normal((b, tq, hq, d))
    return q, k, v, do, q_ids, q_pos, k_ids, k_pos


def _torch_forward(q, k, v, vis, scale):
    """Masked attention with torch ops; rows without a visible key give 0."""
    b, tq, hq, d = q.shape
    grp = hq // k.shape[2]
    kk = k.repeat_interleave(grp, dim=2)          # [B, Tk, Hq, D]
    vv = v.repeat_interleave(grp, dim=2)
    s = torch.einsum("bqhd,bkhd->bhqk", q, kk) * scale
    m = vis[:, None, :, :]                        # [B, 1, Tq, Tk]
    live = m.any(dim=-1, keepdim=True)
    s = torch.where(m, s, torch.full_like(s, -np.inf))
    s = torch.where(live, s, torch.zeros_like(s))   # dead rows: finite, then zeroed
    p = torch.softmax(s, dim=-1) * live
    return torch.einsum("bhqk,bkhd->bqhd", p, vv)


def _vis(q_ids, q_pos, k_ids, k_pos, causal, window):
    return torch.from_numpy(np.stack([oracle.visible(q_ids[b], q_pos[b], k_ids[b], k_pos[b],
                                                     causal, window)
                                      for b in range(q_ids.shape[0])]))


@pytest.mark.parametrize("seed,causal,window,self_attn", [
    (1, True, (-1, -1), True), (2, True, (5, 0), True), (3, False, (-1, -1), False),
    (4, False, (6, 3), False), (5, True, (0, 0), True)])
def test_backward_matches_torch_autograd(seed, causal, window, self_attn):
    q, k, v, do, qi, qp, ki, kp = _case(seed, self_attn=self_attn)
    scale = q.shape[-1] ** -0.5
    tq_, tk_, tv_ = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    vis = _vis(qi, qp, ki, kp, causal, window)
    o = _torch_forward(tq_, tk_, tv_, vis, scale)
    o.backward(torch.tensor(do))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, causal=causal,
                                           window=window)
    np.testing.assert_allclose(dq, tq_.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk_.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv_.grad.numpy(), atol=1e-11, rtol=0)


def test_backward_matches_finite_differences():
    q, k, v, do, qi, qp, ki, kp = _case(11, b=1, tq=9, tk=11, hq=2, hkv=1, d=4)
    kw = dict(causal=False, window=(-1, -1))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, **kw)
    rng = np.random.default_rng(12)
    eps = 1e-6

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, qi, qp, ki, kp, **kw)
        return float((o * do).sum())

    for _ in range(3):
        uq, uk, uv = (rng.standard_normal(x.shape) for x in (q, k, v))
        fd = (loss(q + eps * uq, k + eps * uk, v + eps * uv)
              - loss(q - eps * uq, k - eps * uk, v - eps * uv)) / (2 * eps)
        an = (dq * uq).sum() + (dk * uk).sum() + (dv * uv).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def test_uniform_v_closed_form():
    q, k, v, do, qi, qp, ki, kp = _case(21, self_attn=True)
    v[:] = np.random.default_rng(22).standard_normal((1, 1, v.shape[2], v.shape[3]))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # dV = P^T dO with P from the forward: P = exp(S - LSE) on visible pairs
    o, lse = oracle.attention(q, k, v, qi, qp, ki, kp)
    scale = q.shape[-1] ** -0.5
    grp = q.shape[2] // k.shape[2]
    vis = _vis(qi, qp, ki, kp, True, (-1, -1)).numpy()
    want = np.zeros_like(dv)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            g = h // grp
            s = scale * q[b, :, h] @ k[b, :, g].T
            with np.errstate(invalid="ignore"):
                p = np.where(vis[b], np.exp(s - lse[b, :, h][:, None]), 0.0)
            want[b, :, g] += p.T @ do[b, :, h]
    np.testing.assert_allclose(dv, want, atol=1e-11, rtol=0)


def test_single_visible_key_closed_form():
    q, k, v, do, qi, qp, ki, kp = _case(31, self_attn=True)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, window=(0, 0))
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    grp = q.shape[2] // k.shape[2]
    want = np.zeros_like(dv)
    for b in range(q.shape[0]):
        for t in range(q.shape[1]):
            if qi[b, t] != 0:      # the only key a live token sees is itself
                for h in range(q.shape[2]):
                    want[b, t, h // grp] += do[b, t, h]
    np.testing.assert_allclose(dv, want, atol=1e-12, rtol=0)


def test_invariants():
    q, k, v, do, qi, qp, ki, kp = _case(41, self_attn=True)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, window=(7, 0))
    # a common shift of every key a row sees leaves its softmax unchanged:
    # summed over keys, dK vanishes per (batch row, segment, K/V head)
    for b in range(q.shape[0]):
        for sid in np.unique(qi[b]):
            if sid == 0:
                continue
            sel = ki[b] == sid
            assert np.abs(dk[b, sel].sum(axis=0)).max() < 1e-10
    # padding queries have zero dQ; padding keys get nothing
    assert np.abs(dq[qi == 0]).max(initial=0) == 0 and np.abs(dk[ki == 0]).max(initial=0) == 0
    assert np.abs(dv[ki == 0]).max(initial=0) == 0
    z = oracle.attention_backward(q, k, v, np.zeros_like(do), qi, qp, ki, kp)
    assert all(np.abs(x).max() == 0 for x in z)


def test_sampled_rows_and_keys_equal_full():
    q, k, v, do, qi, qp, ki, kp = _case(51, tq=60, self_attn=True)
    kw = dict(causal=True, window=(9, 0))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qi, qp, ki, kp, **kw)
    rows = [(0, 0), (0, 17), (1, 33), (1, 59)]
    got = oracle.backward_query_rows(q, k, v, do, qi, qp, ki, kp, rows, **kw)
    np.testing.assert_allclose(got, np.stack([dq[b, t] for b, t in rows]), atol=1e-12, rtol=0)
    gk, gv = oracle.backward_key_rows(q, k, v, do, qi, qp, ki, kp, rows, **kw)
    np.testing.assert_allclose(gk, np.stack([dk[b, t] for b, t in rows]), atol=1e-12, rtol=0)
    np.testing.assert_allclose(gv, np.stack([dv[b, t] for b, t in rows]), atol=1e-12, rtol=0)


def test_backward_value_head_dim_differs_torch_autograd():
    """V (and dO) with their own head dim, as with MLA head dimensions."""
    rng = np.random.default_rng(61)
    b, t, hq, hkv, d, dv = 2, 31, 4, 2, 12, 20
    qi, qp = random_layout(rng, b, t, max_segments=3, pad_prob=0.2)
    q = rng.standard_normal((b, t, hq, d))
    k = rng.standard_normal((b, t, hkv, d))
    v = rng.standard_normal((b, t, hkv, dv))
    do = rng.standard_normal((b, t, hq, dv))
    scale = d ** -0.5
    tq_, tk_, tv_ = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    vis = _vis(qi, qp, qi, qp, True, (7, 0))
    o = _torch_forward(tq_, tk_, tv_, vis, scale)
    o.backward(torch.tensor(do))
    dq, dk, dv_ = oracle.attention_backward(q, k, v, do, qi, qp, qi, qp, window=(7, 0))
    assert dv_.shape == v.shape
    np.testing.assert_allclose(dq, tq_.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk_.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv_, tv_.grad.numpy(), atol=1e-11, rtol=0)
    # the sampled forms agree with the full one at a distinct V head dim too
    rows = [(0, 0), (0, 12), (1, 30)]
    gq = oracle.backward_query_rows(q, k, v, do, qi, qp, qi, qp, rows, window=(7, 0))
    np.testing.assert_allclose(gq, np.stack([dq[b_, t_] for b_, t_ in rows]), atol=1e-12, rtol=0)
    gk, gv = oracle.backward_key_rows(q, k, v, do, qi, qp, qi, qp, rows, window=(7, 0))
    assert gv.shape == (len(rows), hkv, dv)
    np.testing.assert_allclose(gk, np.stack([dk[b_, t_] for b_, t_ in rows]), atol=1e-12, rtol=0)
    np.testing.assert_allclose(gv, np.stack([dv_[b_, t_] for b_, t_ in rows]), atol=1e-12, rtol=0)
