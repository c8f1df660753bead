"""Python binding of libringattn (ctypes; argument marshalling only).

Every function here validates shapes, picks dtypes and strides, allocates
outputs with torch on the tensors' device and calls the C ABI declared in
``include/ringattn.h`` on torch's current stream.  All arithmetic happens in
the library's HIP kernels; there is no fallback path: if the shared library
is missing or the tensors are not on an AMD GPU the call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # imported before the library so both share one HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libringattn.so")

RA_BF16, RA_F32 = 0, 1
DUAL_CHUNK, STRIPED = 0, 1
TILE_SKIP, TILE_PARTIAL, TILE_FULL = 0, 1, 2

STATUS = {0: "RA_OK", 1: "RA_ERR_NULL", 2: "RA_ERR_SHAPE", 3: "RA_ERR_DTYPE", 4: "RA_ERR_ALIGN",
          5: "RA_ERR_UNSUPPORTED", 6: "RA_ERR_WORKSPACE", 7: "RA_ERR_ALIAS", 8: "RA_ERR_HIP"}

EXPORTS = ["ra_version", "ra_status_string", "ra_last_error", "ra_check_support", "ra_tile_shape",
           "ra_attn_fwd_workspace_size", "ra_attn_fwd", "ra_attn_fwd_accumulate",
           "ra_classify_tiles", "ra_attn_merge", "ra_reorder", "ra_inverse_reorder",
           "ra_reorder_index", "ra_attn_bwd_workspace_size", "ra_attn_bwd",
           "ra_profile_next_kernel", "ra_attn_fwd_noalloc", "ra_attn_fwd_workspace_parts",
           "ra_attn_fwd_ex"]

# Flags of ra_attn_fwd_ex: the schedule / packed K/V buffer already holds this call's data.
FWD_SCHEDULE_READY, FWD_KV_READY = 1, 2

# Size of the no-allocation forward's per-GPU scratch (RA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 256 << 20


class RingAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "kv_len", "num_q_heads", "num_kv_heads", "head_dim",
        "qkv_dtype", "out_dtype")] + [("scale", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("causal", "window_left", "window_right")] + [
        (n, ctypes.c_int64) for n in (
            "q_batch_stride", "kv_batch_stride", "o_batch_stride", "lse_batch_stride",
            "q_meta_batch_stride", "kv_meta_batch_stride", "q_token_stride", "kv_token_stride",
            "o_token_stride")] + [("v_head_dim", ctypes.c_int32), ("o_split_row", ctypes.c_int32),
                                  ("v_batch_stride", ctypes.c_int64),
                                  ("v_token_stride", ctypes.c_int64),
                                  ("o_split_offset", ctypes.c_int64),
                                  ("lse_split_offset", ctypes.c_int64)]


class Partial(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("o_batch_stride", ctypes.c_int64),
                ("lse_batch_stride", ctypes.c_int64)]


class MergeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq_len", "num_heads", "head_dim", "a_dtype", "b_dtype", "out_dtype")] + [
        (n, ctypes.c_int64) for n in (
            "o_a_batch_stride", "o_b_batch_stride", "o_out_batch_stride",
            "lse_a_batch_stride", "lse_b_batch_stride", "lse_out_batch_stride")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libringattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python __graft_entry__.py build` "
                           "(or blockwise_online_softmax_fwd_amd/build.py)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "ra_version": ([], ctypes.c_char_p),
        "ra_status_string": ([I32], ctypes.c_char_p),
        "ra_last_error": ([], ctypes.c_char_p),
        "ra_check_support": ([ctypes.POINTER(AttnDesc)], I32),
        "ra_tile_shape": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(I32), ctypes.POINTER(I32)], I32),
        "ra_attn_fwd_workspace_size": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ)], I32),
        "ra_attn_fwd": ([ctypes.POINTER(AttnDesc)] + [P] * 9 + [P, SZ, P], I32),
        "ra_attn_fwd_accumulate": ([ctypes.POINTER(AttnDesc)] + [P] * 7 +
                                   [ctypes.POINTER(Partial)] + [P] * 2 + [P, SZ, P], I32),
        "ra_classify_tiles": ([ctypes.POINTER(AttnDesc)] + [P] * 6 + [P, SZ, P], I32),
        "ra_attn_merge": ([ctypes.POINTER(MergeDesc)] + [P] * 6 + [P], I32),
        "ra_reorder": ([P, P, I32, I32, I64, I32, I32, I32, P], I32),
        "ra_inverse_reorder": ([P, P, I32, I32, I64, I32, I32, I32, P], I32),
        "ra_reorder_index": ([I32, I32, I32, I32, I32, P], I32),
        "ra_attn_bwd_workspace_size": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ)], I32),
        "ra_attn_bwd": ([ctypes.POINTER(AttnDesc)] + [P] * 10 + [I32] + [P] * 3 + [P, SZ, P], I32),
        "ra_profile_next_kernel": ([P, P], I32),
        "ra_attn_fwd_noalloc": ([ctypes.POINTER(AttnDesc)] + [P] * 9 + [P], I32),
        "ra_attn_fwd_workspace_parts": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ),
                                         ctypes.POINTER(SZ)], I32),
        "ra_attn_fwd_ex": ([ctypes.POINTER(AttnDesc)] + [P] * 7 + [ctypes.POINTER(Partial)] +
                           [P, P, P, SZ, P, SZ, ctypes.c_uint32, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise RingAttnError(status, load_library().ra_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return RA_BF16
    if dt == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _torch_dtype(code: int):
    return torch.bfloat16 if code == RA_BF16 else torch.float32


def _batch_stride(t, inner_dims: int) -> int:
    """Batch stride of a [B, T, ...] tensor whose non-batch dims are dense."""
    if t.numel() == 0:
        return 0
    expect = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.size(d) > 1 and t.stride(d) != expect:
            raise ValueError(f"tensor of shape {tuple(t.shape)} must be dense below the batch dim")
        expect *= t.size(d)
    return t.stride(0) if t.size(0) > 1 else 0


def _bt_strides(t):
    """(batch stride, token stride) of a [B, T, H, D] tensor whose H and D dims are
    dense (the layouts of the library: BSHD, SBHD, and views into packed K/V or
    Q/K/V buffers).  Size-1 dims report the dense value."""
    if t.dim() != 4:
        raise ValueError("expected a [B, T, H, D] tensor")
    b, n, h, d = t.shape
    if (d > 1 and t.stride(3) != 1) or (h > 1 and t.stride(2) != d):
        raise ValueError(f"tensor of shape {tuple(t.shape)} must have dense heads and head_dim")
    ts = t.stride(1) if n > 1 else h * d
    bs = t.stride(0) if b > 1 else n * ts
    return bs, ts


def _check_meta(q_ids, q_pos, kv_ids, kv_pos):
    """Segment ids and positions: int32 [B, T], tokens contiguous, ids and
    positions of one side sharing a batch stride."""
    for t in (q_ids, q_pos, kv_ids, kv_pos):
        if t.dtype != torch.int32 or t.dim() != 2:
            raise TypeError("segment ids and positions must be int32 [B, T]")
        if t.size(1) > 1 and t.stride(1) != 1:
            raise ValueError("segment ids and positions must be contiguous along the tokens")
    if (_batch_stride(q_pos, 1) != _batch_stride(q_ids, 1)
            or _batch_stride(kv_pos, 1) != _batch_stride(kv_ids, 1)):
        raise ValueError("segment ids and positions must share their batch stride")


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libringattn needs tensors on the GPU")


def version() -> str:
    return load_library().ra_version().decode()


def make_desc(batch, q_len, kv_len, num_q_heads, num_kv_heads, head_dim, qkv_dtype=RA_BF16,
              out_dtype=None, scale=None, causal=True, window=(-1, -1), strides=None) -> AttnDesc:
    d = AttnDesc()
    d.batch, d.q_len, d.kv_len = batch, q_len, kv_len
    d.num_q_heads, d.num_kv_heads, d.head_dim = num_q_heads, num_kv_heads, head_dim
    d.qkv_dtype = qkv_dtype
    d.out_dtype = qkv_dtype if out_dtype is None else out_dtype
    d.scale = float((head_dim ** -0.5 if head_dim > 0 else 1.0) if scale is None else scale)
    d.causal = int(bool(causal))
    d.window_left, d.window_right = int(window[0]), int(window[1])
    if strides:
        for k, v in strides.items():
            setattr(d, k, int(v))
    return d


def check_support(desc: AttnDesc) -> int:
    """0 if supported, else the status code (see ``ra_last_error``)."""
    return load_library().ra_check_support(ctypes.byref(desc))


def tile_shape(desc: AttnDesc):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().ra_tile_shape(ctypes.byref(desc), ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def workspace_size(desc: AttnDesc) -> int:
    n = ctypes.c_size_t()
    _check(load_library().ra_attn_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def workspace_parts(desc: AttnDesc):
    """Bytes of the forward workspace's two parts: ``(schedule, packed K/V)``."""
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().ra_attn_fwd_workspace_parts(ctypes.byref(desc), ctypes.byref(a),
                                                      ctypes.byref(b)))
    return a.value, b.value


def _run_fwd(desc, q, k, v, qi, qp, ki, kp, part, out, lse, workspace, prepared):
    """ra_attn_fwd / ra_attn_fwd_accumulate with one workspace, or ra_attn_fwd_ex
    with ``prepared = (schedule_ws, kv_ws, flags)``."""
    lib = load_library()
    pp = ctypes.byref(part) if part is not None else None
    if prepared is not None:
        sched, kvw, flags = prepared
        need_s, need_k = workspace_parts(desc)
        if sched is None or sched.numel() < need_s or (need_k and (kvw is None or kvw.numel() < need_k)):
            raise ValueError(f"prepared workspaces need {need_s} and {need_k} bytes")
        _check(lib.ra_attn_fwd_ex(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(qi), _ptr(qp), _ptr(ki), _ptr(kp),
            pp, _ptr(out), _ptr(lse), _ptr(sched), ctypes.c_size_t(sched.numel()),
            _ptr(kvw) if kvw is not None else None,
            ctypes.c_size_t(kvw.numel() if kvw is not None else 0), ctypes.c_uint32(flags),
            _stream(q)))
        return
    ws_bytes = workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if part is None:
        _check(lib.ra_attn_fwd(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(qi), _ptr(qp), _ptr(ki), _ptr(kp),
            _ptr(out), _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(q)))
    else:
        _check(lib.ra_attn_fwd_accumulate(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(qi), _ptr(qp), _ptr(ki), _ptr(kp),
            pp, _ptr(out), _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
            _stream(q)))


def _attn_desc(q, k, q_ids, kv_ids, scale, causal, window, out_dtype, o, lse, v=None):
    b, tq, hq, d = q.shape
    tk, hkv = k.shape[1], k.shape[2]
    (qbs, qts), (kbs, kts) = _bt_strides(q), _bt_strides(k)
    strides = {
        "q_batch_stride": qbs, "q_token_stride": qts,
        "kv_batch_stride": kbs, "kv_token_stride": kts,
        "q_meta_batch_stride": _batch_stride(q_ids, 1),
        "kv_meta_batch_stride": _batch_stride(kv_ids, 1),
    }
    if o is not None:
        strides["o_batch_stride"], strides["o_token_stride"] = _bt_strides(o)
    if lse is not None:
        strides["lse_batch_stride"] = _batch_stride(lse, 2)
    if v is not None:
        strides["v_head_dim"] = v.shape[3]
        strides["v_batch_stride"], strides["v_token_stride"] = _bt_strides(v)
    return make_desc(b, tq, tk, hq, hkv, d, _dtype_code(q.dtype), out_dtype, scale, causal,
                     window, strides)


def _apply_split(desc, out, lse, split, tq):
    """Split output: rows >= ``row`` of the call go to ``out_hi`` / ``lse_hi``
    (views with out's and lse's strides) instead of following ``out`` / ``lse``."""
    row, out_hi, lse_hi = split
    if not 0 < row < tq:
        raise ValueError("the split row must lie inside the query rows")
    if (out.shape[1] != row or lse.shape[1] != row or out_hi.shape[1] != tq - row
            or lse_hi.shape[1] != tq - row):
        raise ValueError("out/lse hold the rows below the split, out_hi/lse_hi the rest")
    if out_hi.dtype != out.dtype or _bt_strides(out_hi) != _bt_strides(out) or lse_hi.stride() != lse.stride():
        raise ValueError("the split halves must share dtype and strides")
    ots = _bt_strides(out)[1]
    o_off = out_hi.data_ptr() - out.data_ptr() - row * ots * out.element_size()
    l_off = lse_hi.data_ptr() - lse.data_ptr() - row * lse.shape[2] * 4
    if o_off < 0 or l_off < 0 or o_off % out.element_size() or l_off % 4:
        raise ValueError("the rows above the split must lie after those below it")
    desc.o_split_row = row
    desc.o_split_offset = o_off // out.element_size()
    desc.lse_split_offset = l_off // 4


def attn_fwd(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, *, scale=None,
             causal=True, window=(-1, -1), out_dtype=None, out=None, lse=None, workspace=None,
             split=None, prepared=None):
    """Masked GQA attention forward.  Returns ``(o, lse)``.

    q ``[B,Tq,Hq,D]``, k ``[B,Tk,Hkv,D]``, v ``[B,Tk,Hkv,Dv]`` (bf16 or fp32,
    same dtype; Dv = D, or D = 192 with Dv = 128 for MLA head dims in bf16),
    ids/pos int32 ``[B,T]``.  O is ``[B,Tq,Hq,Dv]``.  ``out``/``lse`` may be
    given (views into larger or packed buffers); otherwise they are allocated.
    ``split=(row, out_hi, lse_hi)``: query rows >= row are written to
    ``out_hi``/``lse_hi`` (placed after ``out``/``lse`` in the same buffers, which
    then hold rows [0, row) only) -- a split output.
    ``prepared=(schedule_ws, kv_ws, flags)``: the workspace in two parts
    (``ra_attn_fwd_ex``; ``flags`` of ``FWD_SCHEDULE_READY`` / ``FWD_KV_READY``
    skip the classification / packing when the buffers already hold them).
    """
    _require_gpu(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.shape[:3] != v.shape[:3]:
        raise ValueError("k and v must have the same batch, length and heads")
    _check_meta(q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos)
    b, tq, hq, d = q.shape
    oc = _dtype_code(q.dtype) if out_dtype is None else _dtype_code(out_dtype)
    if out is None:
        out = torch.empty((b, tq, hq, v.shape[3]), dtype=_torch_dtype(oc), device=q.device)
    elif _dtype_code(out.dtype) != oc:
        raise TypeError("out has the wrong dtype")
    if lse is None:
        lse = torch.empty((b, tq, hq), dtype=torch.float32, device=q.device)
    desc = _attn_desc(q, k, q_segment_ids, kv_segment_ids, scale, causal, window, oc, out, lse, v)
    if split is not None:
        _apply_split(desc, out, lse, split, tq)
    _run_fwd(desc, q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, None,
             out, lse, workspace, prepared)
    return out, lse


def attn_fwd_noalloc(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, *,
                     out, lse, scale=None, causal=True, window=(-1, -1)):
    """``attn_fwd`` through the entry point that allocates nothing: the caller
    passes the outputs ``out`` and ``lse``; the tile lists and packed K/V go
    to the library's per-GPU scratch (``NOALLOC_SCRATCH_BYTES``).  Calls that
    may overlap in time on one GPU must not be made.  Returns ``(out, lse)``."""
    _require_gpu(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, out, lse)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.shape[:3] != v.shape[:3]:
        raise ValueError("k and v must have the same batch, length and heads")
    _check_meta(q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos)
    desc = _attn_desc(q, k, q_segment_ids, kv_segment_ids, scale, causal, window,
                      _dtype_code(out.dtype), out, lse, v)
    _check(load_library().ra_attn_fwd_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(q_segment_ids), _ptr(q_segment_pos),
        _ptr(kv_segment_ids), _ptr(kv_segment_pos), _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def attn_fwd_accumulate(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos,
                        partial_o, partial_lse, *, scale=None, causal=True, window=(-1, -1),
                        out_dtype=None, out=None, lse=None, workspace=None, split=None,
                        prepared=None):
    """Attention forward merged with a running partial ``(partial_o, partial_lse)``
    over other key sets.  ``out``/``lse`` default to the partial itself (in-place
    update); query tiles with no visible pair in this call are then untouched.
    ``split`` and ``prepared`` as in :func:`attn_fwd` (with ``split``,
    ``out``/``lse`` must be given and be separate from the partial).  Returns
    ``(out, lse)``."""
    _require_gpu(q, k, v, partial_o, partial_lse)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.shape[:3] != v.shape[:3]:
        raise ValueError("k and v must have the same batch, length and heads")
    b, tq, hq, d = q.shape
    if tuple(partial_o.shape) != (b, tq, hq, v.shape[3]) or tuple(partial_lse.shape) != (b, tq, hq):
        raise ValueError("the partial must have o's and lse's shapes")
    _check_meta(q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos)
    if partial_lse.dtype != torch.float32:
        raise TypeError("partial lse must be float32")
    if out is None:
        out = partial_o
    if lse is None:
        lse = partial_lse
    oc = _dtype_code(out.dtype) if out_dtype is None else _dtype_code(out_dtype)
    if _dtype_code(out.dtype) != oc:
        raise TypeError("out has the wrong dtype")
    desc = _attn_desc(q, k, q_segment_ids, kv_segment_ids, scale, causal, window, oc, out, lse, v)
    if split is not None:
        _apply_split(desc, out, lse, split, tq)
    part = Partial()
    part.o, part.lse = partial_o.data_ptr(), partial_lse.data_ptr()
    part.dtype = _dtype_code(partial_o.dtype)
    pbs, pts = _bt_strides(partial_o)
    if pts != _bt_strides(out)[1]:
        raise ValueError("the partial must have out's token stride")
    part.o_batch_stride = pbs
    part.lse_batch_stride = _batch_stride(partial_lse, 2)
    _run_fwd(desc, q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, part,
             out, lse, workspace, prepared)
    return out, lse


def bwd_workspace_size(desc: AttnDesc) -> int:
    n = ctypes.c_size_t()
    _check(load_library().ra_attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def attn_bwd(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, o, lse, dout,
             *, scale=None, causal=True, window=(-1, -1), grad_dtype=torch.float32, dq=None,
             dk=None, dv=None, workspace=None):
    """Gradients ``(dq, dk, dv)`` of the masked GQA attention forward.

    q ``[B,Tq,Hq,D]``, k ``[B,Tk,Hkv,D]``, v ``[B,Tk,Hkv,Dv]`` bf16 (Dv = D, or
    the MLA pair D = 192, Dv = 128); ``o``/``lse`` the forward's outputs for
    the same inputs and mask (o ``[B,Tq,Hq,Dv]``, bf16 or fp32); ``dout`` bf16
    with o's shape and strides.  Gradients are ``grad_dtype`` (float32 or
    bfloat16) with the shapes and strides of q, k and v; given buffers are
    overwritten.
    """
    _require_gpu(q, k, v, q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, o, lse, dout)
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("the backward needs bfloat16 q, k and v")
    if dout.dtype != torch.bfloat16:
        raise TypeError("dout must be bfloat16")
    if k.shape[:3] != v.shape[:3]:
        raise ValueError("k and v must have the same batch, length and heads")
    o_shape = tuple(q.shape[:3]) + (v.shape[3],)
    if tuple(o.shape) != o_shape or tuple(dout.shape) != o_shape or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("o and dout must be [B,Tq,Hq,Dv], lse [B,Tq,Hq]")
    if _bt_strides(dout) != _bt_strides(o):
        raise ValueError("dout must have o's batch and token strides")
    _check_meta(q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos)
    gc = _dtype_code(grad_dtype)
    gdt = _torch_dtype(gc)

    def like(t):
        # the library writes a gradient with its input's batch and token strides
        bs, ts = _bt_strides(t)
        return torch.empty_strided(t.shape, (bs, ts, t.shape[3], 1), dtype=gdt, device=t.device)

    if dq is None:
        dq = like(q)
    if dk is None:
        dk = like(k)
    if dv is None:
        dv = like(v)
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.dtype != gdt or t.shape != ref.shape or _bt_strides(t) != _bt_strides(ref):
            raise ValueError("gradient buffers must have grad_dtype and their input's shape and strides")
    desc = _attn_desc(q, k, q_segment_ids, kv_segment_ids, scale, causal, window,
                      _dtype_code(o.dtype), o, lse, v)
    ws_bytes = bwd_workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check(load_library().ra_attn_bwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(q_segment_ids), _ptr(q_segment_pos),
        _ptr(kv_segment_ids), _ptr(kv_segment_pos), _ptr(o), _ptr(lse), _ptr(dout), gc, _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(q)))
    return dq, dk, dv


def profile_next_kernel(start, stop):
    """Arm a pair of ``torch.cuda.Event(enable_timing=True)`` for the next
    forward call on this thread: ``start`` is recorded right before its
    attention kernel and ``stop`` right after it (classification and K/V
    packing fall outside).  ``None, None`` disarms."""
    if start is None and stop is None:
        _check(load_library().ra_profile_next_kernel(None, None))
        return
    for ev in (start, stop):
        if ev.cuda_event == 0:   # torch creates the event on its first record
            ev.record()
    _check(load_library().ra_profile_next_kernel(ctypes.c_void_p(start.cuda_event),
                                                 ctypes.c_void_p(stop.cuda_event)))


def classify_tiles(q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos, *, num_q_heads,
                   num_kv_heads, head_dim=128, dtype=torch.bfloat16, causal=True, window=(-1, -1),
                   workspace=None, v_head_dim=None):
    """Exact tile classes ``int8 [B, nqt, nkt]`` and visible pairs ``int64 [B]``."""
    _require_gpu(q_segment_ids, q_segment_pos, kv_segment_ids, kv_segment_pos)
    b, tq = q_segment_ids.shape
    tk = kv_segment_ids.shape[1]
    desc = make_desc(b, tq, tk, num_q_heads, num_kv_heads, head_dim, _dtype_code(dtype), None,
                     None, causal, window, {
                         "q_meta_batch_stride": _batch_stride(q_segment_ids, 1),
                         "kv_meta_batch_stride": _batch_stride(kv_segment_ids, 1),
                         "v_head_dim": v_head_dim or 0})
    bm, bn = tile_shape(desc)
    nqt, nkt = -(-tq // bm), -(-tk // bn)
    dev = q_segment_ids.device
    classes = torch.empty((b, nqt, nkt), dtype=torch.int8, device=dev)
    pairs = torch.empty((b,), dtype=torch.int64, device=dev)
    ws_bytes = workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(load_library().ra_classify_tiles(
        ctypes.byref(desc), _ptr(q_segment_ids), _ptr(q_segment_pos), _ptr(kv_segment_ids),
        _ptr(kv_segment_pos), _ptr(classes), _ptr(pairs), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(q_segment_ids)))
    return classes, pairs


def attn_merge(o_a, lse_a, o_b, lse_b, *, out=None, lse_out=None, out_dtype=None):
    """Merge two (O, LSE) partials over disjoint key sets.  ``out``/``lse_out``
    may be ``o_a``/``lse_a`` (or the b operands) for in-place accumulation."""
    _require_gpu(o_a, lse_a, o_b, lse_b)
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or o_a.shape[:3] != lse_a.shape:
        raise ValueError("merge operands must have matching [B,T,H,D] / [B,T,H] shapes")
    for t in (lse_a, lse_b):
        if t.dtype != torch.float32:
            raise TypeError("lse must be float32")
    b, t, h, d = o_a.shape
    oc = _dtype_code(o_a.dtype) if out_dtype is None else _dtype_code(out_dtype)
    if out is None:
        out = torch.empty((b, t, h, d), dtype=_torch_dtype(oc), device=o_a.device)
    if lse_out is None:
        lse_out = torch.empty((b, t, h), dtype=torch.float32, device=o_a.device)
    md = MergeDesc()
    md.batch, md.seq_len, md.num_heads, md.head_dim = b, t, h, d
    md.a_dtype, md.b_dtype, md.out_dtype = _dtype_code(o_a.dtype), _dtype_code(o_b.dtype), _dtype_code(out.dtype)
    md.o_a_batch_stride, md.o_b_batch_stride = _batch_stride(o_a, 3), _batch_stride(o_b, 3)
    md.o_out_batch_stride = _batch_stride(out, 3)
    md.lse_a_batch_stride, md.lse_b_batch_stride = _batch_stride(lse_a, 2), _batch_stride(lse_b, 2)
    md.lse_out_batch_stride = _batch_stride(lse_out, 2)
    _check(load_library().ra_attn_merge(ctypes.byref(md), _ptr(o_a), _ptr(lse_a), _ptr(o_b),
                                        _ptr(lse_b), _ptr(out), _ptr(lse_out), _stream(o_a)))
    return out, lse_out


def _kind_code(kind) -> int:
    if kind in ("dual_chunk", DUAL_CHUNK):
        return DUAL_CHUNK
    if kind in ("striped", STRIPED):
        return STRIPED
    raise ValueError(f"unknown reorder kind {kind!r}")


def _reorder(fn_name, x, cp_size, kind, stripe_size, out):
    _require_gpu(x)
    if not x.is_contiguous():
        raise ValueError("reorder needs a contiguous [B, T, ...] tensor")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    b, t = x.shape[0], x.shape[1]
    row_bytes = x.element_size() * (x.numel() // max(1, b * t)) if b * t else x.element_size()
    fn = getattr(load_library(), fn_name)
    _check(fn(_ptr(x), _ptr(out), b, t, row_bytes, cp_size, _kind_code(kind), stripe_size,
              _stream(x)))
    return out


def reorder(x, cp_size, kind="dual_chunk", stripe_size=1, out=None):
    """``out[b, p] = x[b, map(p)]`` along the sequence axis (dim 1)."""
    return _reorder("ra_reorder", x, cp_size, kind, stripe_size, out)


def inverse_reorder(x, cp_size, kind="dual_chunk", stripe_size=1, out=None):
    """``out[b, map(p)] = x[b, p]``: undoes :func:`reorder`."""
    return _reorder("ra_inverse_reorder", x, cp_size, kind, stripe_size, out)


def reorder_index(seq_len, cp_size, kind="dual_chunk", stripe_size=1, inverse=False) -> np.ndarray:
    """The library's map as a host int32 array (computed on the host, no GPU)."""
    out = np.empty(seq_len, dtype=np.int32)
    _check(load_library().ra_reorder_index(seq_len, cp_size, _kind_code(kind), stripe_size,
                                           int(bool(inverse)), out.ctypes.data_as(ctypes.c_void_p)))
    return out
