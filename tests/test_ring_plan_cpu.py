"""Host logic of the ring driver's per-stripe schedule (no GPU)."""

import torch

from blockwise_online_softmax_fwd_amd.ring import _stripe_schedule, needs_reordered_q


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
