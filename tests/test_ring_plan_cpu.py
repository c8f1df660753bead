"""Host logic of the ring driver's per-stripe schedule (no GPU)."""

import torch

import pytest

from blockwise_online_softmax_fwd_amd.ring import RingPlan, _stripe_schedule, needs_reordered_q
from workloads import packed_metadata


def test_stripe_schedule_roles():
    """Each stripe starts at its first step with work and finishes at its last;
    a stripe with no work at all is finished (written empty) at the last step."""
    hp = torch.tensor([[5, 0, 0, 0], [5, 0, 0, 7]])
    sched = _stripe_schedule(hp, 4)
    assert sched[0] == {(True, True): [0], (True, False): [1]}
    assert sched[1] == {} and sched[2] == {}
    assert sched[3] == {(False, True): [1]}
    sched = _stripe_schedule(torch.tensor([[0, 0, 0, 0], [1, 1, 0, 0]]), 4)
    assert sched[0] == {(True, False): [1]} and sched[1] == {(False, True): [1]}
    assert sched[3] == {(True, True): [0]}


def test_q_in_place_only_without_joint_calls():
    """Q needs its reordered copy only when some call covers both stripes."""
    separate = torch.tensor([[[5, 0, 0, 0], [5, 0, 0, 7]], [[4, 3, 0, 0], [4, 0, 0, 0]]] * 2)
    assert not needs_reordered_q(separate, 4)
    joint = torch.tensor([[[5, 2, 0, 0], [5, 2, 0, 0]], [[1, 0, 0, 0], [0, 0, 0, 1]]] * 2)
    assert needs_reordered_q(joint, 4)
    assert needs_reordered_q(None, 4) and needs_reordered_q(torch.ones(4, 4), 4)


def test_plan_refuses_another_layout_or_mask():
    """A plan records the layout and mask it was computed for; using it with
    other ids or positions, another shard count, reorder or mask is refused
    (it would skip blocks that hold visible pairs)."""
    ids, pos = packed_metadata(2, 4096, 4, 768)
    counts = torch.ones((4, 4), dtype=torch.int64)
    plan = RingPlan(counts, ids, pos, 4, "dual_chunk", 1, True, (-1, -1))
    plan.check(ids, pos, 4, "dual_chunk", 1, True, (-1, -1))
    plan.check(ids.clone(), pos.clone(), 4, "dual_chunk", 1, True, (-1, -1))   # same values
    for args in [(8, "dual_chunk", 1, True, (-1, -1)), (4, "striped", 1, True, (-1, -1)),
                 (4, "dual_chunk", 1, False, (-1, -1)), (4, "dual_chunk", 1, True, (100, 0))]:
        with pytest.raises(ValueError):
            plan.check(ids, pos, *args)
    other_ids, other_pos = packed_metadata(2, 4096, 4, 700)
    with pytest.raises(ValueError):
        plan.check(other_ids, other_pos, 4, "dual_chunk", 1, True, (-1, -1))
    shifted = pos.clone()
    shifted[1, 5] += 1
    with pytest.raises(ValueError):
        plan.check(ids, shifted, 4, "dual_chunk", 1, True, (-1, -1))
    # an in-place change of checked tensors is seen too
    ids2 = ids.clone()
    plan.check(ids2, pos, 4, "dual_chunk", 1, True, (-1, -1))
    ids2[0, 0] = 9
    with pytest.raises(ValueError):
        plan.check(ids2, pos, 4, "dual_chunk", 1, True, (-1, -1))
    assert needs_reordered_q(plan, 4)


def test_ring_graph_refuses_before_any_gpu_work():
    """RingGraph checks its plan and the inputs' device before it allocates
    or captures anything."""
    from blockwise_online_softmax_fwd_amd import RingGraph
    ids, pos = packed_metadata(1, 1024, 2, 400)
    q = torch.zeros((1, 1024, 4, 64), dtype=torch.bfloat16)
    k = torch.zeros((1, 1024, 4, 64), dtype=torch.bfloat16)
    plan = RingPlan(torch.ones((2, 2), dtype=torch.int64), ids, pos, 2, "dual_chunk", 1, True,
                    (-1, -1))
    with pytest.raises(TypeError):
        RingGraph(q, k, k, ids, pos, 2, "dual_chunk", 1, plan=plan.counts)
    with pytest.raises(ValueError, match="device tensor"):
        RingGraph(q, k, k, ids, pos, 2, "dual_chunk", 1, plan=plan)
