"""Seeded input generators (values and metadata only; no attention arithmetic).

Values: fp32 N(0, 1) drawn with a seeded ``torch.Generator`` in the order
Q, K, V, then rounded to bf16 with round-to-nearest-even (``Tensor.to``) when
the workload is bf16.  The same host (or device) tensors are handed to both the
HIP path and the oracle, so the two always see identical inputs.

Metadata: the packed layout of the TransformerEngine JAX context-parallel
tutorial, section 1: every slot holds ``valid`` tokens of segment id
``slot + 1`` and then padding tokens with id 0; positions count from 0 through
the whole slot, padding included; the row pattern is tiled over the batch.
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import Workload


def packed_metadata(batch: int, seq_len: int, slots: int, valid_per_slot: int):
    """Return int32 ``(segment_ids, segment_pos)``, each ``[batch, seq_len]`` (host)."""
    if seq_len % slots:
        raise ValueError("seq_len must be a multiple of the slot count")
    slot_len = seq_len // slots
    if not 0 <= valid_per_slot <= slot_len:
        raise ValueError("valid_per_slot out of range")
    ids, pos = [], []
    for s in range(slots):
        ids.append(np.concatenate([np.full(valid_per_slot, s + 1, np.int32),
                                   np.zeros(slot_len - valid_per_slot, np.int32)]))
        pos.append(np.arange(slot_len, dtype=np.int32))
    ids = np.tile(np.concatenate(ids)[None, :], (batch, 1))
    pos = np.tile(np.concatenate(pos)[None, :], (batch, 1))
    return torch.from_numpy(np.ascontiguousarray(ids)), torch.from_numpy(np.ascontiguousarray(pos))


def _dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def random_qkv(batch, q_len, kv_len, hq, hkv, d, dtype="bf16", seed=0, device="cpu", dv=None):
    """Q ``[B,Tq,Hq,D]``, K ``[B,Tk,Hkv,D]`` and V ``[B,Tk,Hkv,Dv]`` (Dv = D unless
    given): N(0,1) drawn in fp32, then cast."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = []
    dv = d if dv is None else dv
    for shape in ((batch, q_len, hq, d), (batch, kv_len, hkv, d), (batch, kv_len, hkv, dv)):
        x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        out.append(x.to(_dtype(dtype)))
    return tuple(out)


def qkv(w: Workload, device="cpu", seed=None):
    """Full-size Q, K, V of a workload (unsplit, original token order)."""
    s = w.seed if seed is None else seed
    return random_qkv(w.batch, w.seq_len, w.seq_len, w.num_q_heads, w.num_kv_heads,
                      w.head_dim, w.dtype, s, device, dv=w.dv)


def random_layout(rng: np.random.Generator, batch: int, seq_len: int, max_segments: int = 4,
                  pad_prob: float = 0.3, pos_offset_max: int = 0):
    """A random packed layout: contiguous runs of segments and padding.

    Each row is cut into random runs; a run is either padding (id 0) or a new
    segment with a fresh id; positions count up from a random offset inside a
    segment and keep counting through padding, as in the packed layout.
    Returns int32 host tensors ``(segment_ids, segment_pos)``.
    """
    ids = np.zeros((batch, seq_len), np.int32)
    pos = np.zeros((batch, seq_len), np.int32)
    for b in range(batch):
        t = 0
        next_id = 1
        while t < seq_len:
            run = int(rng.integers(1, max(2, seq_len // max(1, max_segments)) + 1))
            run = min(run, seq_len - t)
            start = int(rng.integers(0, pos_offset_max + 1)) if pos_offset_max > 0 else 0
            if rng.random() < pad_prob:
                ids[b, t:t + run] = 0
            else:
                ids[b, t:t + run] = next_id
                next_id += 1
            pos[b, t:t + run] = start + np.arange(run, dtype=np.int32)
            t += run
    return torch.from_numpy(ids), torch.from_numpy(pos)
