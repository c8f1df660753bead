"""Full-size workload inputs and row samples shared by the GPU tests.

Inputs are drawn with torch's device generator (seeded per workload) so the
full-size tensors never cross PCIe; the oracle reads the same tensors back.
"""

import numpy as np
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


def stratified_rows(w, rng, tile=32, cp_size=4):
    """One query row per ``tile``-token query tile of every launch, for the
    unsplit call and for both ring layouts of ``cp_size`` shards at once.

    A tile of a dual-chunk launch is ``tile`` consecutive tokens of the
    original order (a dual-chunk stripe is contiguous); a tile of a striped(1)
    launch of rank r is the tokens ``r + cp_size * j`` for ``tile``
    consecutive j, i.e. one residue class of a block of ``cp_size * tile``
    consecutive tokens.  In each such block the residues r are matched to the
    block's ``cp_size`` sub-blocks of ``tile`` tokens by a random permutation
    and one token of residue r is drawn from its sub-block, so every tile of
    both layouts (and of the unsplit call) holds exactly one sampled row.
    Returns sorted ``(batch, token)`` pairs in the original order.
    """
    span = cp_size * tile
    assert w.seq_len % span == 0
    rows = []
    for b in range(w.batch):
        for base in range(0, w.seq_len, span):
            perm = rng.permutation(cp_size)
            for r in range(cp_size):
                sub = base + tile * int(perm[r])
                j = int(rng.integers(tile // cp_size))
                rows.append((b, sub + cp_size * j + r))
    return sorted(rows)


def tiles_covered(rows, order, tile=32):
    """Set of (batch, tile index) of the rows' positions in the reordered
    sequence ``order`` (``order[p]`` = original token at reordered position p)."""
    inv = np.empty_like(order)
    inv[order] = np.arange(len(order))
    return {(b, int(inv[t]) // tile) for b, t in rows}
