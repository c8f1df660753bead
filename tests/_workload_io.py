"""Full-size workload inputs and row samples shared by the GPU tests.

Inputs are drawn with torch's device generator (seeded per workload) so the
full-size tensors never cross PCIe; the oracle reads the same tensors back.
"""

import torch

from workloads import packed_metadata

DEV = "cuda"


def sample_rows(w, rng, extra_positions, n_random=64):
    rows = set()
    for b in range(w.batch):
        for s in range(w.slots):
            base = s * w.slot_len
            for p in extra_positions:
                if 0 <= p < w.slot_len:
                    rows.add((b, base + p))
    for _ in range(n_random):
        rows.add((int(rng.integers(w.batch)), int(rng.integers(w.seq_len))))
    return sorted(rows)


def device_inputs(w, zero_q=False, uniform_v=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(w.seed)
    dt = torch.bfloat16
    q = torch.randn((w.batch, w.seq_len, w.num_q_heads, w.head_dim), generator=g, device=DEV).to(dt)
    k = torch.randn((w.batch, w.seq_len, w.num_kv_heads, w.head_dim), generator=g, device=DEV).to(dt)
    v = torch.randn((w.batch, w.seq_len, w.num_kv_heads, w.dv), generator=g, device=DEV).to(dt)
    if zero_q:
        q.zero_()
    if uniform_v is not None:
        v.copy_(uniform_v.to(DEV, dt)[None, None].expand_as(v))
    ids, pos = packed_metadata(w.batch, w.seq_len, w.slots, w.valid_per_slot)
    return q, k, v, ids.to(DEV), pos.to(DEV)


def closed_form_counts(w, pos_row, ids_row):
    """Visible keys of each query on the packed layouts: min(pos+1, left+1)."""
    p = pos_row.to(torch.float64)
    n = p + 1 if w.window[0] < 0 else torch.clamp(p + 1, max=w.window[0] + 1)
    return torch.where(ids_row != 0, n, torch.zeros_like(n))
