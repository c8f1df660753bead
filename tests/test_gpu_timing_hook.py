"""GPU test of the measurement hook ``ra_profile_next_kernel``: the armed
events bracket the attention kernel inside the forward call, are consumed by
that one call, and leave the results unchanged."""

import pytest
import torch

import blockwise_online_softmax_fwd_amd as bosf
from workloads import packed_metadata, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bosf.load_library()


def test_kernel_events_inside_the_call():
    ids, pos = packed_metadata(2, 2048, 2, 900)
    q, k, v = random_qkv(2, 2048, 2048, 16, 2, 128, "bf16", seed=77)
    args = [t.to(DEV) for t in (q, k, v, ids, pos, ids, pos)]
    ref_o, ref_l = bosf.attn_fwd(*args)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bosf.profile_next_kernel(k0, k1)
    c0.record()
    o, lse = bosf.attn_fwd(*args)
    c1.record()
    torch.cuda.synchronize()
    kernel_ms, call_ms = k0.elapsed_time(k1), c0.elapsed_time(c1)
    print(f"kernel {kernel_ms:.4f} ms inside a {call_ms:.4f} ms call")
    assert 0.0 < kernel_ms <= call_ms
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
    # consumed: the next call does not record the pair again
    bosf.attn_fwd(*args)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == kernel_ms
