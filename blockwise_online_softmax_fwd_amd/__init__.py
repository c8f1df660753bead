"""MI355X-native blockwise online-softmax attention forward (and its backward).

The compute lives in ``libringattn.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/ringattn.h``); :mod:`.ringattn` is its ctypes binding and
:mod:`.ring` the one-GPU ring driver that orders its calls.
"""

from .ringattn import (  # noqa: F401
    DUAL_CHUNK,
    FWD_KV_READY,
    FWD_SCHEDULE_READY,
    NOALLOC_SCRATCH_BYTES,
    STRIPED,
    TILE_FULL,
    TILE_PARTIAL,
    TILE_SKIP,
    RingAttnError,
    attn_bwd,
    attn_fwd,
    attn_fwd_accumulate,
    attn_fwd_noalloc,
    attn_merge,
    bwd_workspace_size,
    check_support,
    classify_tiles,
    inverse_reorder,
    load_library,
    make_desc,
    profile_next_kernel,
    reorder,
    reorder_index,
    tile_shape,
    version,
    workspace_parts,
    workspace_size,
)
from .ring import (RingBuffers, RingGraph, allgather_forward, needs_reordered_q,  # noqa: F401
                   ring_forward, ring_plan)
