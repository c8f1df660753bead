"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function ``include/ringattn.h``
declares, share torch's HIP runtime, and reject every malformed call with the
right status before it touches HIP.  The host copy of the reorder map (the
same function the reorder kernel evaluates) is compared with the oracle.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from blockwise_online_softmax_fwd_amd import ringattn as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, ALIAS = 0, 1, 2, 3, 4, 5, 6, 7


@pytest.fixture(scope="module")
def lib():
    return ra.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ra.EXPORTS) == names


def test_shares_torch_hip_runtime(lib):
    import torch
    torch_lib = os.path.realpath(os.path.join(os.path.dirname(torch.__file__), "lib"))
    maps = open("/proc/self/maps").read()
    hip = {os.path.realpath(l.split()[-1]) for l in maps.splitlines() if "libamdhip64" in l}
    assert hip and all(p.startswith(torch_lib) for p in hip), hip


def test_version_and_strings(lib):
    assert ra.version().startswith("libringattn")
    assert lib.ra_status_string(0) == b"ok"
    assert lib.ra_status_string(8) == b"HIP error"


def _desc(**kw):
    base = dict(batch=2, q_len=100, kv_len=300, num_q_heads=16, num_kv_heads=2, head_dim=128,
                qkv_dtype=ra.RA_BF16)
    base.update(kw)
    extra = {k: base.pop(k) for k in list(base) if k not in (
        "batch", "q_len", "kv_len", "num_q_heads", "num_kv_heads", "head_dim", "qkv_dtype",
        "out_dtype", "scale", "causal", "window")}
    d = ra.make_desc(**base)
    for k, v in extra.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    (dict(qkv_dtype=ra.RA_F32, head_dim=64), OK),
    (dict(batch=0), OK),
    (dict(q_len=0, kv_len=0), OK),
    (dict(num_q_heads=12, num_kv_heads=4), OK),
    (dict(window=(0, 0)), OK),
    (dict(batch=-1), SHAPE),
    (dict(q_len=-5), SHAPE),
    (dict(num_kv_heads=0), SHAPE),
    (dict(num_q_heads=10, num_kv_heads=4), SHAPE),
    (dict(head_dim=96), UNSUP),
    (dict(head_dim=0), SHAPE),
    (dict(qkv_dtype=7), DTYPE),
    (dict(out_dtype=3), DTYPE),
    (dict(scale=0.0), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(scale=float("nan")), SHAPE),
    (dict(window=(-2, 0)), SHAPE),
    (dict(window=(0, -3)), SHAPE),
    (dict(q_batch_stride=-1), SHAPE),
    (dict(kv_batch_stride=5), SHAPE),
    (dict(kv_len=64 * 32768 + 1), UNSUP),
])
def test_check_support(lib, kw, status):
    d = _desc(**kw)
    assert ra.check_support(d) == status
    if status:
        assert lib.ra_last_error().decode()


def test_null_desc(lib):
    assert lib.ra_check_support(None) == NULL
    assert lib.ra_attn_fwd(None, *([None] * 9), None, 0, None) == NULL


def test_profile_hook_arguments(lib):
    """Both events or neither; an armed pair is consumed by the next forward
    call even when that call fails validation (here before any HIP call, so
    the placeholder handles are never touched)."""
    fake = ctypes.c_void_p(0x1000)
    assert lib.ra_profile_next_kernel(fake, None) == NULL
    assert lib.ra_profile_next_kernel(None, fake) == NULL
    assert lib.ra_profile_next_kernel(None, None) == OK
    assert lib.ra_profile_next_kernel(fake, ctypes.c_void_p(0x2000)) == OK
    assert lib.ra_attn_fwd(None, *([None] * 9), None, 0, None) == NULL
    assert lib.ra_profile_next_kernel(None, None) == OK


@pytest.mark.parametrize("hq,hkv,bm", [(16, 2, 32), (128, 8, 32), (64, 8, 32), (8, 2, 64),
                                       (4, 1, 64), (3, 1, 256), (12, 1, 64), (6, 3, 128)])
def test_tile_shape_bf16(hq, hkv, bm):
    assert ra.tile_shape(_desc(num_q_heads=hq, num_kv_heads=hkv)) == (bm, 64)


def test_tile_shape_f32():
    assert ra.tile_shape(_desc(qkv_dtype=ra.RA_F32, num_q_heads=4, num_kv_heads=4,
                               head_dim=64)) == (64, 32)


def test_workspace_size_grows_with_tiles():
    small = ra.workspace_size(_desc(q_len=64, kv_len=64))
    big = ra.workspace_size(_desc(q_len=4096, kv_len=4096))
    assert 0 < small < big
    # list of nqt x nkt 4-byte entries per batch row dominates
    assert big >= 2 * (4096 // 32) * (4096 // 64) * 4


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def _p(off=0):
    return ctypes.c_void_p(FAKE + off)


def _fwd(lib, d, ws_bytes=1 << 30, **over):
    args = dict(q=_p(0), k=_p(1 << 32), v=_p(2 << 32), qid=_p(3 << 32), qpos=_p(4 << 32),
                kid=_p(5 << 32), kpos=_p(6 << 32), o=_p(7 << 32), lse=_p(8 << 32), ws=_p(9 << 32))
    args.update(over)
    return lib.ra_attn_fwd(ctypes.byref(d), args["q"], args["k"], args["v"], args["qid"],
                           args["qpos"], args["kid"], args["kpos"], args["o"], args["lse"],
                           args["ws"], ctypes.c_size_t(ws_bytes), None)


def test_fwd_rejects_null_pointers(lib):
    d = _desc()
    for name in ("q", "k", "v", "o", "lse", "qid", "qpos", "kid", "kpos"):
        assert _fwd(lib, d, **{name: None}) == NULL, name
    assert _fwd(lib, d, ws=None) == WS


def test_fwd_rejects_misalignment(lib):
    d = _desc()
    for name in ("q", "k", "v", "o"):
        assert _fwd(lib, d, **{name: _p(8)}) == ALIGN, name
    assert _fwd(lib, d, lse=_p((8 << 32) + 2)) == ALIGN
    assert _fwd(lib, d, qid=_p((3 << 32) + 1)) == ALIGN
    assert _fwd(lib, d, ws=_p((9 << 32) + 16)) == ALIGN
    d2 = _desc(q_batch_stride=100 * 16 * 128 + 4)  # 8-byte stride remainder in bf16
    assert _fwd(lib, d2) == ALIGN


def test_fwd_rejects_small_workspace(lib):
    d = _desc()
    need = ra.workspace_size(d)
    assert _fwd(lib, d, ws_bytes=need - 1) == WS


def test_fwd_rejects_aliasing(lib):
    d = _desc()
    assert _fwd(lib, d, o=_p(0)) == ALIAS                 # o == q
    assert _fwd(lib, d, o=_p(1 << 32)) == ALIAS           # o == k
    assert _fwd(lib, d, lse=_p((7 << 32) + 4096)) == ALIAS  # lse inside o


def test_workspace_and_metadata_aliasing(lib):
    """The workspace (overwritten by the classification and packing kernels)
    must not overlap any argument, and the outputs must not overlap the
    segment ids or positions: each such call is refused before any HIP call."""
    d = _desc()
    need = ra.workspace_size(d)
    for name in ("q", "k", "v", "qid", "qpos", "kid", "kpos", "o", "lse"):
        base = {"q": 0, "k": 1, "v": 2, "qid": 3, "qpos": 4, "kid": 5, "kpos": 6, "o": 7,
                "lse": 8}[name]
        assert _fwd(lib, d, ws=_p(base << 32), ws_bytes=need) == ALIAS, name
    # the workspace's whole extent counts: one starting below lse and reaching into it
    assert _fwd(lib, d, ws=_p((8 << 32) - 256), ws_bytes=need) == ALIAS
    assert _fwd(lib, d, o=_p(3 << 32)) == ALIAS          # o over the query ids
    assert _fwd(lib, d, lse=_p(6 << 32)) == ALIAS        # lse over the key positions
    # accumulate: the workspace over the partial
    part = ra.Partial()
    part.o, part.lse, part.dtype = FAKE + (10 << 32), FAKE + (11 << 32), ra.RA_F32
    for ws in (10, 11):
        assert lib.ra_attn_fwd_accumulate(ctypes.byref(d), _p(0), _p(1 << 32), _p(2 << 32),
                                          _p(3 << 32), _p(4 << 32), _p(5 << 32), _p(6 << 32),
                                          ctypes.byref(part), _p(7 << 32), _p(8 << 32),
                                          _p(ws << 32), ctypes.c_size_t(need), None) == ALIAS
    # classification: outputs over the metadata, workspace over an output
    c = ctypes.c_void_p(FAKE + (12 << 32))
    n = ctypes.c_void_p(FAKE + (13 << 32))

    def classify(classes, pairs, ws):
        return lib.ra_classify_tiles(ctypes.byref(d), _p(3 << 32), _p(4 << 32), _p(5 << 32),
                                     _p(6 << 32), classes, pairs, ws, ctypes.c_size_t(need), None)
    assert classify(_p(3 << 32), n, _p(9 << 32)) == ALIAS
    assert classify(c, _p(6 << 32), _p(9 << 32)) == ALIAS
    assert classify(c, n, _p(12 << 32)) == ALIAS
    assert classify(c, c, _p(9 << 32)) == ALIAS
    # backward: gradients over the metadata, workspace over a gradient or input
    assert _bwd(lib, d, dq=_p(3 << 32)) == ALIAS
    assert _bwd(lib, d, dk=_p(5 << 32)) == ALIAS
    for base in (0, 7, 10, 11, 12, 13, 4):
        assert _bwd(lib, d, ws=_p(base << 32)) == ALIAS, base


def test_noalloc_scratch_limit_and_validation(lib):
    """The no-allocation forward's scratch size is the header's, and a call
    that needs more scratch is refused with a clear error before any HIP
    call; argument checks are ra_attn_fwd's."""
    text = open(HEADER).read()
    m = re.search(r"#define RA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ra.NOALLOC_SCRATCH_BYTES

    def call(d, **over):
        args = dict(q=_p(0), k=_p(1 << 32), v=_p(2 << 32), qid=_p(3 << 32), qpos=_p(4 << 32),
                    kid=_p(5 << 32), kpos=_p(6 << 32), o=_p(7 << 32), lse=_p(8 << 32))
        args.update(over)
        return lib.ra_attn_fwd_noalloc(ctypes.byref(d), args["q"], args["k"], args["v"],
                                       args["qid"], args["qpos"], args["kid"], args["kpos"],
                                       args["o"], args["lse"], None)
    big = _desc(batch=2, q_len=32768, kv_len=65536, num_q_heads=64, num_kv_heads=8)
    assert ra.workspace_size(big) > ra.NOALLOC_SCRATCH_BYTES
    assert call(big) == WS
    msg = lib.ra_last_error().decode()
    assert "scratch" in msg and str(ra.NOALLOC_SCRATCH_BYTES) in msg
    assert lib.ra_attn_fwd_noalloc(None, *([None] * 9), None) == NULL
    d = _desc()
    assert ra.workspace_size(d) <= ra.NOALLOC_SCRATCH_BYTES
    assert call(d, q=None) == NULL
    assert call(d, o=_p(8)) == ALIGN
    assert call(d, o=_p(0)) == ALIAS
    assert call(_desc(head_dim=96)) == UNSUP


def test_split_workspace_parts_and_validation(lib):
    """ra_attn_fwd_workspace_parts splits ra_attn_fwd_workspace_size's bytes in two
    (tile lists; packed K/V, empty for fp32), and ra_attn_fwd_ex checks both
    buffers (size, alignment, overlaps with each other and with every argument)
    and its flags before any HIP call."""
    for kw in ({}, dict(qkv_dtype=ra.RA_F32, head_dim=64), dict(q_len=4096, kv_len=4096),
               dict(head_dim=192, v_head_dim=128)):
        d = _desc(**kw)
        sb, kb = ra.workspace_parts(d)
        assert sb + kb == ra.workspace_size(d) and sb > 0
        assert (kb == 0) == (d.qkv_dtype == ra.RA_F32)
    d = _desc()
    sb, kb = ra.workspace_parts(d)

    def call(sched=_p(9 << 32), sbytes=sb, kv=_p(10 << 32), kbytes=kb, flags=0, partial=None, **over):
        args = dict(q=_p(0), k=_p(1 << 32), v=_p(2 << 32), qid=_p(3 << 32), qpos=_p(4 << 32),
                    kid=_p(5 << 32), kpos=_p(6 << 32), o=_p(7 << 32), lse=_p(8 << 32))
        args.update(over)
        return lib.ra_attn_fwd_ex(ctypes.byref(d), args["q"], args["k"], args["v"], args["qid"],
                                  args["qpos"], args["kid"], args["kpos"], partial, args["o"],
                                  args["lse"], sched, ctypes.c_size_t(sbytes), kv,
                                  ctypes.c_size_t(kbytes), ctypes.c_uint32(flags), None)
    assert lib.ra_attn_fwd_ex(None, *([None] * 7), None, None, None, None, 0, None, 0, 0,
                              None) == NULL
    assert call(sched=None) == WS
    assert call(sbytes=sb - 1) == WS
    assert call(kv=None) == WS
    assert call(kbytes=kb - 1) == WS
    assert call(sched=_p((9 << 32) + 16)) == ALIGN
    assert call(kv=_p((10 << 32) + 128)) == ALIGN
    assert call(flags=4) == SHAPE
    assert call(kv=_p((9 << 32) + ((sb + 255) // 256) * 256 - 256)) == ALIAS   # kv starts in sched
    assert call(sched=_p(0)) == ALIAS                                          # sched over q
    assert call(kv=_p(5 << 32)) == ALIAS                                       # kv over key ids
    assert call(q=None) == NULL
    assert call(o=_p(0)) == ALIAS
    part = ra.Partial()
    part.o, part.lse, part.dtype = FAKE + (11 << 32), FAKE + (12 << 32), ra.RA_F32
    assert call(partial=ctypes.byref(part), kv=_p(11 << 32)) == ALIAS           # kv over the partial
    bad = ra.Partial()
    bad.o, bad.lse, bad.dtype = FAKE + (11 << 32), None, ra.RA_F32
    assert call(partial=ctypes.byref(bad)) == NULL
    d32 = _desc(qkv_dtype=ra.RA_F32, head_dim=64)
    d = d32
    assert call(sbytes=ra.workspace_parts(d32)[0] - 1, kv=None, kbytes=0) == WS


def test_accumulate_validation(lib):
    d = _desc()
    part = ra.Partial()
    part.o, part.lse, part.dtype = FAKE + (10 << 32), FAKE + (11 << 32), ra.RA_F32

    def call(pp, o=_p(7 << 32), lse=_p(8 << 32)):
        return lib.ra_attn_fwd_accumulate(ctypes.byref(d), _p(0), _p(1 << 32), _p(2 << 32),
                                          _p(3 << 32), _p(4 << 32), _p(5 << 32), _p(6 << 32),
                                          pp, o, lse, _p(9 << 32), ctypes.c_size_t(1 << 30), None)
    assert call(None) == NULL
    bad = ra.Partial()
    bad.o, bad.lse, bad.dtype = FAKE + (10 << 32), None, ra.RA_F32
    assert call(ctypes.byref(bad)) == NULL
    bad.lse, bad.dtype = FAKE + (11 << 32), 9
    assert call(ctypes.byref(bad)) == DTYPE
    bad.dtype, bad.o = ra.RA_F32, FAKE + (10 << 32) + 8
    assert call(ctypes.byref(bad)) == ALIGN
    bad.o, bad.o_batch_stride = FAKE + (10 << 32), 3
    assert call(ctypes.byref(bad)) == SHAPE
    # o overlapping the partial without being it (shifted, or other dtype)
    assert call(ctypes.byref(part), o=_p((10 << 32) + 256)) == ALIAS
    d.out_dtype = ra.RA_BF16
    assert call(ctypes.byref(part), o=_p(10 << 32), lse=_p(11 << 32)) == ALIAS


def test_split_output_validation(lib):
    """A split output (rows >= o_split_row moved o_split_offset / lse_split_offset
    further on) is checked before any launch: its row inside the query rows, the
    offsets >= 0 and aligned, each batch row's extent inside its batch stride,
    no overlap of the extent with an input, no in-place partial, and only the
    forward outputs may be split."""
    L = 16 * 128                                    # one o row (elements), q_len 100
    ok = dict(o_split_row=50, o_split_offset=300 * L, lse_split_offset=300 * 16,
              o_batch_stride=1000 * L, lse_batch_stride=1000 * 16)
    assert ra.check_support(_desc(**ok)) == OK
    for bad, st in [(dict(o_split_row=100), SHAPE), (dict(o_split_row=-1), SHAPE),
                    (dict(o_split_row=0), SHAPE),                    # offsets without a row
                    (dict(o_split_offset=-L), SHAPE),
                    (dict(o_batch_stride=300 * L), SHAPE),          # extent past the batch stride
                    (dict(lse_batch_stride=300 * 16), SHAPE),
                    (dict(o_token_stride=L // 2, o_batch_stride=L // 2 * 100), SHAPE)]:
        assert ra.check_support(_desc(**{**ok, **bad})) == st, bad
    assert _fwd(lib, _desc(**{**ok, "o_split_offset": 300 * L + 4})) == ALIGN   # 8 bytes in bf16
    # q sits in the gap between o's rows below the split (200 KB) and those
    # moved 300 rows further on
    assert _fwd(lib, _desc(**ok), o=_p(-(512 << 10))) == ALIAS
    # in place is refused with a split
    d = _desc(**ok)
    d.out_dtype = ra.RA_F32
    part = ra.Partial()
    part.o, part.lse, part.dtype = FAKE + (7 << 32), FAKE + (8 << 32), ra.RA_F32
    part.o_batch_stride, part.lse_batch_stride = 1000 * L, 1000 * 16
    assert lib.ra_attn_fwd_accumulate(ctypes.byref(d), _p(0), _p(1 << 32), _p(2 << 32),
                                      _p(3 << 32), _p(4 << 32), _p(5 << 32), _p(6 << 32),
                                      ctypes.byref(part), _p(7 << 32), _p(8 << 32), _p(9 << 32),
                                      ctypes.c_size_t(1 << 30), None) == ALIAS
    # only the forward's output can be split
    assert _bwd(lib, _desc(**ok)) == UNSUP
    c = (ctypes.c_int8 * 8)()
    n = (ctypes.c_int64 * 2)()
    assert lib.ra_classify_tiles(ctypes.byref(_desc(**ok)), _p(3 << 32), _p(4 << 32), _p(5 << 32),
                                 _p(6 << 32), c, n, _p(9 << 32), ctypes.c_size_t(1 << 30),
                                 None) == UNSUP


def _merge(lib, md, **over):
    args = dict(oa=_p(0), la=_p(1 << 32), ob=_p(2 << 32), lb=_p(3 << 32), oo=_p(4 << 32),
                lo=_p(5 << 32))
    args.update(over)
    return lib.ra_attn_merge(ctypes.byref(md), args["oa"], args["la"], args["ob"], args["lb"],
                             args["oo"], args["lo"], None)


def _mdesc(**kw):
    md = ra.MergeDesc()
    md.batch, md.seq_len, md.num_heads, md.head_dim = 2, 64, 8, 128
    md.a_dtype = md.b_dtype = md.out_dtype = ra.RA_F32
    for k, v in kw.items():
        setattr(md, k, v)
    return md


def test_merge_validation(lib):
    assert lib.ra_attn_merge(None, *([None] * 7)) == NULL
    assert _merge(lib, _mdesc(head_dim=32)) == UNSUP
    assert _merge(lib, _mdesc(a_dtype=5)) == DTYPE
    assert _merge(lib, _mdesc(batch=-1)) == SHAPE
    assert _merge(lib, _mdesc(o_a_batch_stride=7)) == SHAPE
    assert _merge(lib, _mdesc(), oa=None) == NULL
    assert _merge(lib, _mdesc(), oa=_p(4)) == ALIGN
    assert _merge(lib, _mdesc(), lb=_p((3 << 32) + 1)) == ALIGN
    # in-place on a with identical layout is fine only at validation level; a shifted
    # overlap is not
    assert _merge(lib, _mdesc(), oo=_p(16)) == ALIAS
    assert _merge(lib, _mdesc(out_dtype=ra.RA_BF16), oo=_p(0)) == ALIAS
    assert _merge(lib, _mdesc(), lo=_p((1 << 32) + 4)) == ALIAS
    assert _merge(lib, _mdesc(batch=0)) == OK


def test_reorder_validation(lib):
    f = lib.ra_reorder
    assert f(_p(0), _p(1 << 32), 2, 100, 4, 4, ra.DUAL_CHUNK, 1, None) == SHAPE   # 100 % 8
    assert f(_p(0), _p(1 << 32), 2, 96, 4, 4, ra.STRIPED, 5, None) == SHAPE       # 96 % 20
    assert f(_p(0), _p(1 << 32), 2, 96, 0, 4, ra.DUAL_CHUNK, 1, None) == SHAPE
    assert f(_p(0), _p(1 << 32), 2, 96, 4, 0, ra.DUAL_CHUNK, 1, None) == SHAPE
    assert f(_p(0), _p(1 << 32), 2, 96, 4, 4, 9, 1, None) == SHAPE
    assert f(None, _p(1 << 32), 2, 96, 4, 4, ra.DUAL_CHUNK, 1, None) == NULL
    assert f(_p(0), _p(100), 2, 96, 4, 4, ra.DUAL_CHUNK, 1, None) == ALIAS
    assert lib.ra_inverse_reorder(_p(0), _p(0), 1, 8, 4, 4, ra.DUAL_CHUNK, 1, None) == ALIAS
    assert f(_p(0), _p(1 << 32), 0, 96, 4, 4, ra.DUAL_CHUNK, 1, None) == OK       # empty


@pytest.mark.parametrize("t,r,kind,s", [(16, 4, "dual_chunk", 1), (4096, 4, "dual_chunk", 1),
                                        (65536, 4, "dual_chunk", 1), (96, 3, "striped", 8),
                                        (4096, 4, "striped", 1), (65536, 4, "striped", 512),
                                        (24, 1, "striped", 3), (12, 1, "dual_chunk", 1)])
def test_reorder_index_matches_oracle(t, r, kind, s):
    m = ra.reorder_index(t, r, kind, s)
    ref = oracle.reorder_map(t, r, kind, s)
    assert np.array_equal(m, ref)
    inv = ra.reorder_index(t, r, kind, s, inverse=True)
    assert np.array_equal(inv, oracle.inverse_map(ref))


def _bwd(lib, d, ws_bytes=1 << 34, grad=ra.RA_F32, **over):
    args = dict(q=_p(0), k=_p(1 << 32), v=_p(2 << 32), qid=_p(3 << 32), qpos=_p(4 << 32),
                kid=_p(5 << 32), kpos=_p(6 << 32), o=_p(7 << 32), lse=_p(8 << 32),
                dout=_p(10 << 32), dq=_p(11 << 32), dk=_p(12 << 32), dv=_p(13 << 32),
                ws=_p(16 << 32))
    args.update(over)
    return lib.ra_attn_bwd(ctypes.byref(d), args["q"], args["k"], args["v"], args["qid"],
                           args["qpos"], args["kid"], args["kpos"], args["o"], args["lse"],
                           args["dout"], grad, args["dq"], args["dk"], args["dv"], args["ws"],
                           ctypes.c_size_t(ws_bytes), None)


def test_bwd_workspace_size():
    d = _desc(q_len=4096, kv_len=4096)
    n = ra.bwd_workspace_size(d)
    # packed Q and dO rows alone (2 batch rows x Tq x Hq rows of 136 bf16 each, 128 of
    # data plus padding), plus the packed K/V tiles (K, V and K^T per key tile)
    q_rows = 2 * 2 * 4096 * 16 * 136 * 2
    kv_tiles = 2 * 2 * (4096 // 64) * (64 * 136 * 2 * 2 + 128 * 72 * 2)
    assert n > q_rows + kv_tiles
    assert ra.bwd_workspace_size(_desc(q_len=64, kv_len=64)) < n
    d32 = _desc(qkv_dtype=ra.RA_F32, head_dim=64)
    with pytest.raises(ra.RingAttnError, match="RA_ERR_UNSUPPORTED"):
        ra.bwd_workspace_size(d32)
    with pytest.raises(ra.RingAttnError, match="RA_ERR_UNSUPPORTED"):
        ra.bwd_workspace_size(_desc(q_len=32 * 32768 + 1))


def test_bwd_validation(lib):
    d = _desc()
    assert lib.ra_attn_bwd(None, *([None] * 10), 0, *([None] * 4), 0, None) == NULL
    for name in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "qid", "kpos"):
        assert _bwd(lib, d, **{name: None}) == NULL, name
    assert _bwd(lib, d, ws=None) == WS
    assert _bwd(lib, d, ws_bytes=ra.bwd_workspace_size(d) - 1) == WS
    assert _bwd(lib, d, grad=5) == DTYPE
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        assert _bwd(lib, d, **{name: _p((14 << 32) + 8)}) == ALIGN, name
    assert _bwd(lib, d, lse=_p((8 << 32) + 2)) == ALIGN
    assert _bwd(lib, d, ws=_p((16 << 32) + 64)) == ALIGN
    assert _bwd(lib, _desc(qkv_dtype=ra.RA_F32)) == UNSUP
    assert _bwd(lib, _desc(head_dim=80)) == UNSUP
    # gradients overlapping an input or each other
    assert _bwd(lib, d, dq=_p(0)) == ALIAS
    assert _bwd(lib, d, dk=_p((2 << 32) + 4096)) == ALIAS
    assert _bwd(lib, d, dv=_p(12 << 32)) == ALIAS
    assert _bwd(lib, d, dq=_p((10 << 32) + 16)) == ALIAS
    # empty problems launch nothing and succeed
    assert _bwd(lib, _desc(batch=0)) == OK
    assert _bwd(lib, _desc(q_len=0, kv_len=0), ws=None, ws_bytes=0) == OK


def test_layout_strides_validation(lib):
    hd_q, hd_k = 16 * 128, 2 * 128          # Hq*D, Hkv*D of _desc()
    # packed K/V (T2HD): token stride 2*Hkv*D, v half a row after k
    d = _desc(kv_token_stride=2 * hd_k)
    assert ra.check_support(d) == OK
    # sequence-major (SBHD): batch stride H*D, token stride B*H*D
    d = _desc(q_token_stride=2 * hd_q, q_batch_stride=hd_q, o_token_stride=2 * hd_q,
              o_batch_stride=hd_q)
    assert ra.check_support(d) == OK
    # rows that would overlap
    assert ra.check_support(_desc(q_token_stride=hd_q - 8)) == SHAPE
    assert ra.check_support(_desc(q_token_stride=2 * hd_q, q_batch_stride=hd_q + 8)) == SHAPE
    assert ra.check_support(_desc(kv_token_stride=-8)) == SHAPE
    # token strides must keep 16-byte alignment
    assert _fwd(lib, _desc(q_token_stride=hd_q + 4)) == ALIGN
    assert _bwd(lib, _desc(kv_token_stride=2 * hd_k + 4)) == ALIGN


def test_bwd_packed_gradients_are_not_aliases(lib):
    hd_k = 2 * 128
    d = _desc(kv_token_stride=2 * hd_k, kv_batch_stride=300 * 2 * hd_k)
    base = 12 << 32
    # dk and dv side by side in one packed buffer pass the alias checks (the call
    # then stops at the missing workspace, before any HIP call)
    assert _bwd(lib, d, ws=None, dk=_p(base), dv=_p(base + hd_k * 4)) == WS
    # shifted by less than a row: overlap
    assert _bwd(lib, d, ws=None, dk=_p(base), dv=_p(base + 16)) == ALIAS
    # dq rows side by side with dk, dv at equal strides (packed Q/K/V gradients)
    dq3 = _desc(q_len=300, num_q_heads=2, num_kv_heads=2, q_token_stride=6 * 128,
                kv_token_stride=6 * 128, q_batch_stride=300 * 6 * 128,
                kv_batch_stride=300 * 6 * 128)
    assert _bwd(lib, dq3, ws=None, dq=_p(base), dk=_p(base + 256 * 4),
                dv=_p(base + 512 * 4)) == WS
    assert _bwd(lib, dq3, ws=None, dq=_p(base), dk=_p(base + 128 * 4),
                dv=_p(base + 512 * 4)) == ALIAS


def test_bwd_mla_alias_spans(lib):
    """With MLA head dims V, O, dO and dV rows are 128 wide per head: separate
    buffers pass, and dk and dv side by side in one packed K/V gradient buffer
    (rows of 2 x (192 + 128) elements) pass unless they overlap."""
    d = _desc(head_dim=192, v_head_dim=128, kv_len=300)
    assert _bwd(lib, d, ws=None) == WS
    row = 2 * (192 + 128)
    dp = _desc(head_dim=192, v_head_dim=128, kv_len=300, kv_token_stride=row,
               kv_batch_stride=300 * row, v_token_stride=row, v_batch_stride=300 * row)
    base = 12 << 32
    assert _bwd(lib, dp, ws=None, dk=_p(base), dv=_p(base + 2 * 192 * 4)) == WS
    assert _bwd(lib, dp, ws=None, dk=_p(base), dv=_p(base + 2 * 192 * 4 - 16)) == ALIAS


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=192, v_head_dim=128), OK),
    (dict(head_dim=128, v_head_dim=128), OK),
    (dict(head_dim=64, v_head_dim=0), OK),
    (dict(head_dim=192), UNSUP),                       # v_head_dim 0 means 192
    (dict(head_dim=128, v_head_dim=64), UNSUP),
    (dict(head_dim=192, v_head_dim=128, qkv_dtype=ra.RA_F32), UNSUP),
    (dict(v_head_dim=-1), SHAPE),
    (dict(o_split_row=100), SHAPE),                    # split row must be below q_len
    (dict(head_dim=192, v_head_dim=128, v_token_stride=2 * 128 - 8), SHAPE),
])
def test_value_head_dim_support(lib, kw, status):
    assert ra.check_support(_desc(**kw)) == status


def test_mla_workspaces(lib):
    """MLA head dims (192 / 128) are accepted by the forward and the backward
    (bf16); their workspaces are larger than at 128 / 128; fp32 is refused."""
    d = _desc(head_dim=192, v_head_dim=128)
    assert ra.workspace_size(d) > ra.workspace_size(_desc())
    assert ra.bwd_workspace_size(d) > ra.bwd_workspace_size(_desc())
    with pytest.raises(ra.RingAttnError, match="RA_ERR_UNSUPPORTED"):
        ra.bwd_workspace_size(_desc(head_dim=192, v_head_dim=128, qkv_dtype=ra.RA_F32))
    with pytest.raises(ra.RingAttnError, match="RA_ERR_UNSUPPORTED"):
        ra.bwd_workspace_size(_desc(head_dim=128, v_head_dim=64))
