// C-ABI front end of libringattn: argument validation (host only, before any
// HIP call), workspace carving and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "internal.h"
#include "reorder_map.h"
#include "ringattn.h"

namespace {

thread_local std::string g_last_error;
// Event pair armed by ra_profile_next_kernel for this thread's next forward call.
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

ra_status fail(ra_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ra_status hip_fail(hipError_t e, const char *what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t dtype_size(int32_t dt) { return dt == RA_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dt) { return dt == RA_BF16 || dt == RA_F32; }

constexpr int64_t kMaxKeyTiles = 32768;  // class bytes of one query tile fit in LDS

struct Resolved {
  int64_t q_bs, kv_bs, o_bs, lse_bs, qm_bs, km_bs;
  int64_t q_ts, kv_ts, o_ts;  // token strides (elements)
  int64_t v_bs, v_ts;         // V's strides
  int32_t dv;                 // head dim of V and O
  int32_t bm, bn, nqt, nkt, nt;
  int32_t split;              // split row of o / lse (0: none)
  int64_t o_soff, lse_soff;   // their extra offsets (elements)
};

int64_t pick(int64_t given, int64_t dense) { return given == 0 ? dense : given; }

// True if B x T rows of L elements at batch stride bs and token stride ts never
// overlap, with one stride nesting the other (the layouts the header lists).
bool nested(int64_t B, int64_t T, int64_t L, int64_t bs, int64_t ts) {
  if (B <= 0 || T <= 0 || L <= 0) return true;
  if (B == 1 && T == 1) return true;
  if (B == 1) return ts >= L;
  if (T == 1) return bs >= L;
  if (bs >= ts) return ts >= L && bs >= (T - 1) * ts + L;
  return bs >= L && ts >= (B - 1) * bs + L;
}

ra_status check_desc(const ra_attn_desc *d, Resolved *r) {
  if (!d) return fail(RA_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->q_len < 0 || d->kv_len < 0)
    return fail(RA_ERR_SHAPE, "batch, q_len and kv_len must be >= 0 (got %d, %d, %d)", d->batch,
                d->q_len, d->kv_len);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(RA_ERR_SHAPE, "head counts must be >= 1 (got %d, %d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads)
    return fail(RA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim <= 0) return fail(RA_ERR_SHAPE, "head_dim must be > 0 (got %d)", d->head_dim);
  if (!dtype_ok(d->qkv_dtype)) return fail(RA_ERR_DTYPE, "unknown qkv_dtype %d", d->qkv_dtype);
  if (!dtype_ok(d->out_dtype)) return fail(RA_ERR_DTYPE, "unknown out_dtype %d", d->out_dtype);
  if (d->v_head_dim < 0) return fail(RA_ERR_SHAPE, "v_head_dim must be >= 0");
  r->dv = d->v_head_dim ? d->v_head_dim : d->head_dim;
  {
    const bool same = r->dv == d->head_dim && (d->head_dim == 64 || d->head_dim == 128);
    const bool mla = d->head_dim == 192 && r->dv == 128 && d->qkv_dtype == RA_BF16;
    if (!same && !mla)
      return fail(RA_ERR_UNSUPPORTED,
                  "head dims (%d, %d) not supported: (64, 64), (128, 128) or bf16 (192, 128)",
                  d->head_dim, r->dv);
  }
  if (!(d->scale > 0.0f) || !isfinite(d->scale))
    return fail(RA_ERR_SHAPE, "scale must be finite and > 0");
  if (d->causal != 0 && d->causal != 1) return fail(RA_ERR_SHAPE, "causal must be 0 or 1");
  if (d->window_left < -1 || d->window_right < -1)
    return fail(RA_ERR_SHAPE, "window sizes must be -1 or >= 0 (got %d, %d)", d->window_left,
                d->window_right);
  const int64_t B = d->batch, Tq = d->q_len, Tk = d->kv_len, Hq = d->num_q_heads,
                Hkv = d->num_kv_heads, D = d->head_dim;
  const int64_t DV = r->dv;
  const int64_t strides[11] = {d->q_batch_stride,   d->kv_batch_stride,     d->o_batch_stride,
                               d->lse_batch_stride, d->q_meta_batch_stride, d->kv_meta_batch_stride,
                               d->q_token_stride,   d->kv_token_stride,     d->o_token_stride,
                               d->v_batch_stride,   d->v_token_stride};
  for (int i = 0; i < 11; ++i)
    if (strides[i] < 0) return fail(RA_ERR_SHAPE, "batch and token strides must be >= 0");
  r->q_ts = pick(d->q_token_stride, Hq * D);
  r->kv_ts = pick(d->kv_token_stride, Hkv * D);
  r->o_ts = pick(d->o_token_stride, Hq * DV);
  r->q_bs = pick(d->q_batch_stride, Tq * r->q_ts);
  r->kv_bs = pick(d->kv_batch_stride, Tk * r->kv_ts);
  r->o_bs = pick(d->o_batch_stride, Tq * r->o_ts);
  // V follows K's strides unless its head dim differs or its own are given.
  r->v_ts = pick(d->v_token_stride, DV == D ? r->kv_ts : Hkv * DV);
  r->v_bs = pick(d->v_batch_stride, DV == D && d->v_token_stride == 0 ? r->kv_bs : Tk * r->v_ts);
  r->lse_bs = pick(d->lse_batch_stride, Tq * Hq);
  r->qm_bs = pick(d->q_meta_batch_stride, Tq);
  r->km_bs = pick(d->kv_meta_batch_stride, Tk);
  if (!nested(B, Tq, Hq * D, r->q_bs, r->q_ts) || !nested(B, Tq, Hq * DV, r->o_bs, r->o_ts) ||
      !nested(B, Tk, Hkv * D, r->kv_bs, r->kv_ts) || !nested(B, Tk, Hkv * DV, r->v_bs, r->v_ts))
    return fail(RA_ERR_SHAPE, "q, k, v or o strides let two (batch, token) rows overlap");
  if (B > 1 && (r->lse_bs < Tq * Hq || r->qm_bs < Tq || r->km_bs < Tk))
    return fail(RA_ERR_SHAPE, "a batch stride is smaller than one batch row");
  if (d->o_split_row < 0 || d->o_split_offset < 0 || d->lse_split_offset < 0)
    return fail(RA_ERR_SHAPE, "o_split_row and the split offsets must be >= 0");
  r->split = d->o_split_row;
  r->o_soff = d->o_split_offset;
  r->lse_soff = d->lse_split_offset;
  if (r->split == 0 && (r->o_soff != 0 || r->lse_soff != 0))
    return fail(RA_ERR_SHAPE, "split offsets given without o_split_row");
  if (r->split > 0) {
    if (r->split >= Tq)
      return fail(RA_ERR_SHAPE, "o_split_row %d must be below q_len %d", r->split, d->q_len);
    if (r->o_ts < Hq * DV)
      return fail(RA_ERR_SHAPE, "a split output needs an o token stride of at least Hq*Dv");
    if (B > 1 && (r->o_bs < (Tq - 1) * r->o_ts + r->o_soff + Hq * DV ||
                  r->lse_bs < Tq * Hq + r->lse_soff))
      return fail(RA_ERR_SHAPE, "a split output's batch row extends past its batch stride");
  }
  if (d->qkv_dtype == RA_BF16) {
    r->nt = ra::bf16_token_subtiles(d->num_q_heads / d->num_kv_heads);
    r->bm = 32 * r->nt;
    r->bn = ra::kBnBf16;
  } else {
    r->nt = 0;
    r->bm = ra::kBmF32;
    r->bn = ra::kBnF32;
  }
  const int64_t nqt = (Tq + r->bm - 1) / r->bm, nkt = (Tk + r->bn - 1) / r->bn;
  if (nkt > kMaxKeyTiles)
    return fail(RA_ERR_UNSUPPORTED, "kv_len %lld exceeds %lld key tiles of %d tokens",
                (long long)Tk, (long long)kMaxKeyTiles, r->bn);
  if (B * Hq * nqt >= (int64_t)1 << 31)
    return fail(RA_ERR_UNSUPPORTED, "too many query tiles for one launch");
  r->nqt = (int32_t)nqt;
  r->nkt = (int32_t)nkt;
  return RA_OK;
}

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

size_t span_bytes(int64_t batch, int64_t bs, int64_t row_elems, size_t es) {
  if (batch <= 0 || row_elems <= 0) return 0;
  return (size_t)((batch - 1) * bs + row_elems) * es;
}

// Bytes from the first to one past the last element of a [B, T, L] tensor at
// batch stride bs and token stride ts (elements of size es).
size_t span_bytes2(int64_t batch, int64_t tokens, int64_t L, int64_t bs, int64_t ts, size_t es) {
  if (batch <= 0 || tokens <= 0 || L <= 0) return 0;
  return (size_t)((batch - 1) * bs + (tokens - 1) * ts + L) * es;
}

// Overlap of two [B, T, L] tensors that share their batch and token strides
// (bytes: sb, st; rows of la and lb bytes, Ta and Tb tokens), as when rows of
// several tensors sit side by side in one packed buffer.  Exact when the outer
// stride is a multiple of the inner one; otherwise the spans are compared.
bool rows_overlap(const void *a, int64_t Ta, int64_t la, const void *b, int64_t Tb, int64_t lb,
                  int64_t batch, int64_t sb, int64_t st) {
  if (!a || !b || batch <= 0 || Ta <= 0 || Tb <= 0 || la <= 0 || lb <= 0) return false;
  if ((uintptr_t)a > (uintptr_t)b) {
    const void *tp = a; a = b; b = tp;
    int64_t t = Ta; Ta = Tb; Tb = t;
    t = la; la = lb; lb = t;
  }
  const int64_t d = (int64_t)((uintptr_t)b - (uintptr_t)a);
  if (d >= (batch - 1) * sb + (Ta - 1) * st + la) return false;
  const int64_t T = Ta > Tb ? Ta : Tb;
  const int64_t inner = batch > 1 && T > 1 ? (sb < st ? sb : st) : (T > 1 ? st : sb);
  const int64_t outer = sb < st ? st : sb;
  if (inner <= 0 || (batch > 1 && T > 1 && outer % inner)) return true;
  const int64_t r = d % inner;
  return !(r >= la && r + lb <= inner);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A buffer and its extent in bytes, for the overlap checks.
struct Span {
  const void *p;
  size_t n;
};

// True if any of the n spans overlaps [x, x + xn).
bool overlaps_any(const void *x, size_t xn, const Span *spans, int n) {
  for (int i = 0; i < n; ++i)
    if (overlaps(x, xn, spans[i].p, spans[i].n)) return true;
  return false;
}

// Extents of the four int32 metadata buffers [B, T] at their batch strides.
struct MetaSpans {
  Span s[4];
};
MetaSpans meta_spans(const ra_attn_desc *d, const int64_t qm_bs, const int64_t km_bs,
                     const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                     const int32_t *kpos) {
  const size_t qn = span_bytes(d->batch, qm_bs, d->q_len, 4);
  const size_t kn = span_bytes(d->batch, km_bs, d->kv_len, 4);
  return MetaSpans{{{qid, qn}, {qpos, qn}, {kid, kn}, {kpos, kn}}};
}

ra_status check_meta(const ra_attn_desc *d, const Resolved &r, const int32_t *qid,
                     const int32_t *qpos, const int32_t *kid, const int32_t *kpos) {
  if (d->batch > 0 && d->q_len > 0 && (!qid || !qpos))
    return fail(RA_ERR_NULL, "query segment ids / positions are NULL");
  if (d->batch > 0 && d->kv_len > 0 && (!kid || !kpos))
    return fail(RA_ERR_NULL, "key segment ids / positions are NULL");
  if (!aligned(qid, 4) || !aligned(qpos, 4) || !aligned(kid, 4) || !aligned(kpos, 4))
    return fail(RA_ERR_ALIGN, "segment metadata must be 4-byte aligned");
  (void)r;
  return RA_OK;
}

ra::WorkspaceLayout layout_of(const ra_attn_desc *d, const Resolved &r) {
  const int32_t pd = d->qkv_dtype == RA_BF16 ? d->head_dim : 0;
  return ra::workspace_layout(d->batch, r.nqt, r.nkt, d->num_kv_heads, pd, pd ? r.dv : 0);
}

ra_status check_workspace(const ra_attn_desc *d, const Resolved &r, const void *ws,
                          size_t ws_bytes) {
  const ra::WorkspaceLayout L = layout_of(d, r);
  if (L.total > 0 && !ws) return fail(RA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (ws_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  if (!aligned(ws, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  return RA_OK;
}

ra::Schedule carve(void *ws, const ra::WorkspaceLayout &L) {
  char *base = (char *)ws;
  ra::Schedule s;
  s.qsum = (ra::TileSum *)(base + L.qsum);
  s.ksum = (ra::TileSum *)(base + L.ksum);
  s.count = (int32_t *)(base + L.count);
  s.pairs = (int64_t *)(base + L.pairs);
  s.list = (uint32_t *)(base + L.list);
  return s;
}

ra::MaskParams mask_of(const ra_attn_desc *d) {
  ra::MaskParams m;
  m.causal = d->causal;
  m.wl = d->window_left;
  m.wr = d->window_right;
  return m;
}

ra_status run_schedule(const ra_attn_desc *d, const Resolved &r, const ra::Schedule &s,
                       const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                       const int32_t *kpos, int8_t *classes, hipStream_t st) {
  hipError_t e = ra::launch_summaries(qid, qpos, r.qm_bs, d->batch, d->q_len, r.bm, r.nqt, s.qsum, st);
  if (e != hipSuccess) return hip_fail(e, "tile summaries (queries)");
  e = ra::launch_summaries(kid, kpos, r.km_bs, d->batch, d->kv_len, r.bn, r.nkt, s.ksum, st);
  if (e != hipSuccess) return hip_fail(e, "tile summaries (keys)");
  e = ra::launch_classify(s, qid, qpos, kid, kpos, r.qm_bs, r.km_bs, d->batch, d->q_len, d->kv_len,
                          r.bm, r.bn, r.nqt, r.nkt, mask_of(d), classes, st);
  if (e != hipSuccess) return hip_fail(e, "tile classification");
  return RA_OK;
}

}  // namespace

extern "C" {

const char *ra_version(void) { return "libringattn 0.2.0 (gfx950)"; }

const char *ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK: return "ok";
    case RA_ERR_NULL: return "null pointer";
    case RA_ERR_SHAPE: return "bad shape, stride or window";
    case RA_ERR_DTYPE: return "bad dtype";
    case RA_ERR_ALIGN: return "misaligned pointer or stride";
    case RA_ERR_UNSUPPORTED: return "unsupported configuration";
    case RA_ERR_WORKSPACE: return "workspace missing or too small";
    case RA_ERR_ALIAS: return "overlapping buffers";
    case RA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *ra_last_error(void) { return g_last_error.c_str(); }

ra_status ra_check_support(const ra_attn_desc *desc) {
  Resolved r;
  return check_desc(desc, &r);
}

ra_status ra_tile_shape(const ra_attn_desc *desc, int32_t *bm, int32_t *bn) {
  Resolved r;
  const ra_status st = check_desc(desc, &r);
  if (st != RA_OK) return st;
  if (!bm || !bn) return fail(RA_ERR_NULL, "output pointer is NULL");
  *bm = r.bm;
  *bn = r.bn;
  return RA_OK;
}

ra_status ra_attn_fwd_workspace_size(const ra_attn_desc *desc, size_t *bytes) {
  Resolved r;
  const ra_status st = check_desc(desc, &r);
  if (st != RA_OK) return st;
  if (!bytes) return fail(RA_ERR_NULL, "bytes is NULL");
  *bytes = layout_of(desc, r).total;
  return RA_OK;
}

}  // extern "C"

namespace {

// Scratch of the no-allocation forward: one copy per GPU, reserved when the
// library's code is loaded onto that GPU and held until the process ends.
// Host code never uses this name as an address (on the host it is only a
// stand-in); it uses the per-device pointer that hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device.
ra_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RA_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p % 256) != 0)
      return fail(RA_ERR_HIP, "scratch of device %d has no usable address", dev);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RA_OK;
}

// Where a forward call's workspace comes from: one caller-owned buffer (tile
// lists followed by the packed K/V), this device's scratch, or the two parts
// in separate caller-owned buffers (with flags saying which already hold
// this call's data).
enum class WsMode { kContiguous, kScratch, kSplit };

struct FwdWorkspace {
  WsMode mode;
  void *ws;              // contiguous: the buffer; split: the schedule part
  size_t bytes;
  void *kv;              // split: the packed K/V part
  size_t kv_bytes;
  uint32_t flags;        // split: RA_FWD_* reuse flags
};

ra_status attn_fwd_impl(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                        const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                        const int32_t *kpos, const ra_partial *acc, void *o, float *lse,
                        FwdWorkspace w, ra_stream_t stream) {
  // an armed profiling pair belongs to this call, whatever its outcome
  const hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  Resolved r;
  ra_status st = check_desc(d, &r);
  if (st != RA_OK) return st;
  const bool has_q = d->batch > 0 && d->q_len > 0;
  const bool has_k = d->batch > 0 && d->kv_len > 0;
  if (has_q && (!q || !o || !lse)) return fail(RA_ERR_NULL, "q, o or lse is NULL");
  if (has_k && (!k || !v)) return fail(RA_ERR_NULL, "k or v is NULL");
  st = check_meta(d, r, qid, qpos, kid, kpos);
  if (st != RA_OK) return st;
  const size_t es = dtype_size(d->qkv_dtype), os = dtype_size(d->out_dtype);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(RA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if ((r.q_bs * es) % 16 || (r.kv_bs * es) % 16 || (r.o_bs * os) % 16 || (r.q_ts * es) % 16 ||
      (r.kv_ts * es) % 16 || (r.o_ts * os) % 16 || (r.v_bs * es) % 16 || (r.v_ts * es) % 16)
    return fail(RA_ERR_ALIGN, "batch and token strides of q, k, v and o must be multiples of 16 bytes");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  const int64_t D = d->head_dim;
  const int64_t B = d->batch, Tq = d->q_len, Tk = d->kv_len;
  const int64_t Lq = (int64_t)d->num_q_heads * D, Lk = (int64_t)d->num_kv_heads * D;
  const int64_t Lo = (int64_t)d->num_q_heads * r.dv, Lv = (int64_t)d->num_kv_heads * r.dv;
  const size_t q_span = span_bytes2(B, Tq, Lq, r.q_bs, r.q_ts, es);
  const size_t kv_span = span_bytes2(B, Tk, Lk, r.kv_bs, r.kv_ts, es);
  const size_t v_span = span_bytes2(B, Tk, Lv, r.v_bs, r.v_ts, es);
  // a split output's extent includes the gap before its moved rows
  const size_t o_span = span_bytes2(B, Tq, Lo, r.o_bs, r.o_ts, os) + (size_t)r.o_soff * os;
  const size_t l_span = span_bytes(d->batch, r.lse_bs, (int64_t)d->q_len * d->num_q_heads, 4) +
                        (size_t)r.lse_soff * 4;
  if (r.split > 0 && (r.o_soff * (int64_t)os) % 16)
    return fail(RA_ERR_ALIGN, "o_split_offset must be a multiple of 16 bytes");
  if (overlaps(o, o_span, q, q_span) || overlaps(o, o_span, k, kv_span) ||
      overlaps(o, o_span, v, v_span) || overlaps(lse, l_span, o, o_span) ||
      overlaps(lse, l_span, q, q_span) || overlaps(lse, l_span, k, kv_span) ||
      overlaps(lse, l_span, v, v_span))
    return fail(RA_ERR_ALIAS, "o / lse overlap an input or each other");
  int64_t acc_o_bs = 0, acc_lse_bs = 0;
  bool in_place = false;
  Span acc_span{nullptr, 0}, acc_lspan{nullptr, 0};
  if (acc) {
    if (!dtype_ok(acc->dtype)) return fail(RA_ERR_DTYPE, "unknown partial dtype %d", acc->dtype);
    if (acc->o_batch_stride < 0 || acc->lse_batch_stride < 0)
      return fail(RA_ERR_SHAPE, "partial batch strides must be >= 0");
    const int64_t rows = (int64_t)d->q_len * d->num_q_heads;
    acc_o_bs = pick(acc->o_batch_stride, Tq * r.o_ts);
    acc_lse_bs = pick(acc->lse_batch_stride, rows);
    if (!nested(B, Tq, Lo, acc_o_bs, r.o_ts) || (d->batch > 1 && acc_lse_bs < rows))
      return fail(RA_ERR_SHAPE, "a partial batch stride is smaller than one batch row");
    if (has_q && (!acc->o || !acc->lse)) return fail(RA_ERR_NULL, "partial o or lse is NULL");
    const size_t as = dtype_size(acc->dtype);
    if (!aligned(acc->o, 16) || (acc_o_bs * as) % 16 || !aligned(acc->lse, 4))
      return fail(RA_ERR_ALIGN, "partial o must be 16-byte aligned (lse 4-byte)");
    const size_t a_span = span_bytes2(B, Tq, Lo, acc_o_bs, r.o_ts, as);
    const size_t al_span = span_bytes(d->batch, acc_lse_bs, rows, 4);
    const bool same_o = acc->o == o && acc->dtype == d->out_dtype && acc_o_bs == r.o_bs;
    const bool same_l = acc->lse == lse && acc_lse_bs == r.lse_bs;
    in_place = same_o && same_l && r.split == 0;
    if (!in_place && (overlaps(o, o_span, acc->o, a_span) || overlaps(lse, l_span, acc->lse, al_span) ||
                      overlaps(o, o_span, acc->lse, al_span) || overlaps(lse, l_span, acc->o, a_span)))
      return fail(RA_ERR_ALIAS, "o / lse overlap the partial without being it");
    acc_span = Span{acc->o, a_span};
    acc_lspan = Span{acc->lse, al_span};
  }
  const MetaSpans ms = meta_spans(d, r.qm_bs, r.km_bs, qid, qpos, kid, kpos);
  if (overlaps_any(o, o_span, ms.s, 4) || overlaps_any(lse, l_span, ms.s, 4))
    return fail(RA_ERR_ALIAS, "o / lse overlap the segment ids or positions");
  if (!has_q) return RA_OK;
  const ra::WorkspaceLayout L = layout_of(d, r);
  const size_t sched_need = L.kpack, kv_need = L.total - L.kpack;
  // sched: tile summaries and lists (offsets of L below kpack); kvp: the
  // packed K/V tiles (offsets of L from kpack on, shifted to start at 0)
  char *sched = nullptr, *kvp = nullptr;
  const Span used[11] = {{q, q_span}, {k, kv_span}, {v, v_span}, {o, o_span}, {lse, l_span},
                         acc_span, acc_lspan, ms.s[0], ms.s[1], ms.s[2], ms.s[3]};
  if (w.mode == WsMode::kSplit) {
    if (sched_need > 0 && !w.ws)
      return fail(RA_ERR_WORKSPACE, "schedule workspace is NULL (%zu bytes needed)", sched_need);
    if (w.bytes < sched_need)
      return fail(RA_ERR_WORKSPACE, "schedule workspace has %zu bytes, %zu needed", w.bytes,
                  sched_need);
    if (kv_need > 0 && !w.kv)
      return fail(RA_ERR_WORKSPACE, "K/V workspace is NULL (%zu bytes needed)", kv_need);
    if (w.kv_bytes < kv_need)
      return fail(RA_ERR_WORKSPACE, "K/V workspace has %zu bytes, %zu needed", w.kv_bytes,
                  kv_need);
    if (!aligned(w.ws, 256) || !aligned(w.kv, 256))
      return fail(RA_ERR_ALIGN, "workspaces must be 256-byte aligned");
    if (w.flags & ~(uint32_t)(RA_FWD_SCHEDULE_READY | RA_FWD_KV_READY))
      return fail(RA_ERR_SHAPE, "unknown flags 0x%x", w.flags);
    if (overlaps_any(w.ws, sched_need, used, 11) || overlaps_any(w.kv, kv_need, used, 11))
      return fail(RA_ERR_ALIAS, "a workspace overlaps an input or output");
    if (overlaps(w.ws, sched_need, w.kv, kv_need))
      return fail(RA_ERR_ALIAS, "the schedule and K/V workspaces overlap");
    sched = (char *)w.ws;
    kvp = (char *)w.kv;
  } else {
    void *workspace = w.ws;
    size_t workspace_bytes = w.bytes;
    if (w.mode == WsMode::kScratch) {
      // the no-allocation entry point: the workspace is this device's scratch
      if (L.total > RA_NOALLOC_SCRATCH_BYTES)
        return fail(RA_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; the no-allocation forward holds %zu "
                    "(use ra_attn_fwd with a caller-owned workspace)",
                    L.total, (size_t)RA_NOALLOC_SCRATCH_BYTES);
      st = scratch_of_current_device(&workspace);
      if (st != RA_OK) return st;
      workspace_bytes = RA_NOALLOC_SCRATCH_BYTES;
    }
    st = check_workspace(d, r, workspace, workspace_bytes);
    if (st != RA_OK) return st;
    if (overlaps_any(workspace, L.total, used, 11))
      return fail(RA_ERR_ALIAS, "the workspace overlaps an input or output");
    sched = (char *)workspace;
    kvp = (char *)workspace + L.kpack;
  }
  const bool schedule_ready = w.mode == WsMode::kSplit && (w.flags & RA_FWD_SCHEDULE_READY);
  const bool kv_ready = w.mode == WsMode::kSplit && (w.flags & RA_FWD_KV_READY);

  hipStream_t s = (hipStream_t)stream;
  const ra::Schedule sch = carve(sched, L);
  if (!schedule_ready) {
    st = run_schedule(d, r, sch, qid, qpos, kid, kpos, nullptr, s);
    if (st != RA_OK) return st;
  }

  ra::AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.qid = qid;
  p.qpos = qpos;
  p.kid = kid;
  p.kpos = kpos;
  p.o = o;
  p.lse = lse;
  p.list = sch.list;
  p.count = sch.count;
  p.q_bs = r.q_bs;
  p.kv_bs = r.kv_bs;
  p.o_bs = r.o_bs;
  p.lse_bs = r.lse_bs;
  p.q_ts = r.q_ts;
  p.kv_ts = r.kv_ts;
  p.o_ts = r.o_ts;
  p.v_bs = r.v_bs;
  p.v_ts = r.v_ts;
  p.qm_bs = r.qm_bs;
  p.km_bs = r.km_bs;
  p.batch = d->batch;
  p.tq = d->q_len;
  p.tk = d->kv_len;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.nqt = r.nqt;
  p.nkt = r.nkt;
  p.scale = d->scale;
  p.scale_log2 = d->scale * 1.4426950408889634f;
  p.mask = mask_of(d);
  p.acc_o = acc ? acc->o : nullptr;
  p.acc_lse = acc ? acc->lse : nullptr;
  p.acc_o_bs = acc_o_bs;
  p.acc_lse_bs = acc_lse_bs;
  p.acc_mode = acc ? (acc->dtype == RA_BF16 ? 2 : 1) : 0;
  p.acc_in_place = in_place ? 1 : 0;
  p.o_split = r.split > 0 ? r.split : INT32_MAX;
  p.o_split_off = r.o_soff;
  p.lse_split_off = r.lse_soff;
  p.kpack = kvp;
  p.vpack = kvp + (L.vpack - L.kpack);
  p.mpack = (const int32_t *)(kvp + (L.mpack - L.kpack));
  if (d->qkv_dtype == RA_BF16 && d->kv_len > 0 && !kv_ready) {
    ra::PackParams pk;
    pk.k = k;
    pk.v = v;
    pk.kid = kid;
    pk.kpos = kpos;
    pk.kpack = kvp;
    pk.vpack = kvp + (L.vpack - L.kpack);
    pk.mpack = (int32_t *)(kvp + (L.mpack - L.kpack));
    pk.kv_bs = r.kv_bs;
    pk.kv_ts = r.kv_ts;
    pk.v_bs = r.v_bs;
    pk.v_ts = r.v_ts;
    pk.km_bs = r.km_bs;
    pk.batch = d->batch;
    pk.tk = d->kv_len;
    pk.hkv = d->num_kv_heads;
    pk.nkt = r.nkt;
    const hipError_t pe = ra::launch_pack_kv(pk, d->head_dim, r.dv, s);
    if (pe != hipSuccess) return hip_fail(pe, "K/V tile packing");
  }
  const bool out_bf16 = d->out_dtype == RA_BF16;
  if (ev0) {
    const hipError_t ee = hipEventRecord(ev0, s);
    if (ee != hipSuccess) return hip_fail(ee, "profiling start event");
  }
  const hipError_t e = d->qkv_dtype == RA_BF16
                           ? ra::launch_attn_bf16(p, d->head_dim, r.dv, r.nt, out_bf16, s)
                           : ra::launch_attn_f32(p, d->head_dim, out_bf16, s);
  if (e != hipSuccess) return hip_fail(e, "attention forward");
  if (ev1) {
    const hipError_t ee = hipEventRecord(ev1, s);
    if (ee != hipSuccess) return hip_fail(ee, "profiling stop event");
  }
  return RA_OK;
}

}  // namespace

extern "C" {

ra_status ra_attn_fwd(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                      const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                      const int32_t *kpos, void *o, float *lse, void *workspace,
                      size_t workspace_bytes, ra_stream_t stream) {
  return attn_fwd_impl(d, q, k, v, qid, qpos, kid, kpos, nullptr, o, lse,
                       FwdWorkspace{WsMode::kContiguous, workspace, workspace_bytes, nullptr, 0, 0},
                       stream);
}

ra_status ra_attn_fwd_accumulate(const ra_attn_desc *d, const void *q, const void *k,
                                 const void *v, const int32_t *qid, const int32_t *qpos,
                                 const int32_t *kid, const int32_t *kpos,
                                 const ra_partial *partial, void *o, float *lse, void *workspace,
                                 size_t workspace_bytes, ra_stream_t stream) {
  if (!partial) return fail(RA_ERR_NULL, "partial is NULL");
  return attn_fwd_impl(d, q, k, v, qid, qpos, kid, kpos, partial, o, lse,
                       FwdWorkspace{WsMode::kContiguous, workspace, workspace_bytes, nullptr, 0, 0},
                       stream);
}

ra_status ra_attn_fwd_workspace_parts(const ra_attn_desc *desc, size_t *schedule_bytes,
                                      size_t *kv_bytes) {
  Resolved r;
  const ra_status st = check_desc(desc, &r);
  if (st != RA_OK) return st;
  if (!schedule_bytes || !kv_bytes) return fail(RA_ERR_NULL, "output pointer is NULL");
  const ra::WorkspaceLayout L = layout_of(desc, r);
  *schedule_bytes = L.kpack;
  *kv_bytes = L.total - L.kpack;
  return RA_OK;
}

ra_status ra_attn_fwd_ex(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                         const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                         const int32_t *kpos, const ra_partial *partial, void *o, float *lse,
                         void *schedule_ws, size_t schedule_bytes, void *kv_ws, size_t kv_bytes,
                         uint32_t flags, ra_stream_t stream) {
  return attn_fwd_impl(d, q, k, v, qid, qpos, kid, kpos, partial, o, lse,
                       FwdWorkspace{WsMode::kSplit, schedule_ws, schedule_bytes, kv_ws, kv_bytes,
                                    flags},
                       stream);
}

ra_status ra_attn_fwd_noalloc(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                              const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                              const int32_t *kpos, void *o, float *lse, ra_stream_t stream) {
  return attn_fwd_impl(d, q, k, v, qid, qpos, kid, kpos, nullptr, o, lse,
                       FwdWorkspace{WsMode::kScratch, nullptr, 0, nullptr, 0, 0}, stream);
}

ra_status ra_profile_next_kernel(ra_event_t start, ra_event_t stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(RA_ERR_NULL, "profiling events: pass both or neither");
  g_prof_start = (hipEvent_t)start;
  g_prof_stop = (hipEvent_t)stop;
  return RA_OK;
}

ra_status ra_classify_tiles(const ra_attn_desc *d, const int32_t *qid, const int32_t *qpos,
                            const int32_t *kid, const int32_t *kpos, int8_t *classes,
                            int64_t *visible_pairs, void *workspace, size_t workspace_bytes,
                            ra_stream_t stream) {
  Resolved r;
  ra_status st = check_desc(d, &r);
  if (st != RA_OK) return st;
  if (r.split != 0) return fail(RA_ERR_UNSUPPORTED, "o_split_row applies to the forward's output only");
  st = check_meta(d, r, qid, qpos, kid, kpos);
  if (st != RA_OK) return st;
  if (!aligned(visible_pairs, 8)) return fail(RA_ERR_ALIGN, "visible_pairs must be 8-byte aligned");
  if (d->batch == 0) return RA_OK;
  st = check_workspace(d, r, workspace, workspace_bytes);
  if (st != RA_OK) return st;
  {
    const MetaSpans ms = meta_spans(d, r.qm_bs, r.km_bs, qid, qpos, kid, kpos);
    const size_t cn = (size_t)d->batch * r.nqt * r.nkt, pn = (size_t)d->batch * 8;
    if (overlaps_any(classes, cn, ms.s, 4) || overlaps_any(visible_pairs, pn, ms.s, 4) ||
        overlaps(classes, cn, visible_pairs, pn))
      return fail(RA_ERR_ALIAS, "classes / visible_pairs overlap the metadata or each other");
    const Span used[6] = {{classes, cn}, {visible_pairs, pn}, ms.s[0], ms.s[1], ms.s[2], ms.s[3]};
    if (overlaps_any(workspace, layout_of(d, r).total, used, 6))
      return fail(RA_ERR_ALIAS, "the workspace overlaps an input or output");
  }
  hipStream_t s = (hipStream_t)stream;
  const ra::Schedule sch = carve(workspace, layout_of(d, r));
  st = run_schedule(d, r, sch, qid, qpos, kid, kpos, classes, s);
  if (st != RA_OK) return st;
  if (visible_pairs) {
    const hipError_t e = ra::launch_pair_sums(sch.pairs, d->batch, r.nqt, visible_pairs, s);
    if (e != hipSuccess) return hip_fail(e, "visible pair sums");
  }
  return RA_OK;
}

ra_status ra_attn_merge(const ra_merge_desc *d, const void *o_a, const float *lse_a,
                        const void *o_b, const float *lse_b, void *o_out, float *lse_out,
                        ra_stream_t stream) {
  if (!d) return fail(RA_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0 || d->num_heads < 1)
    return fail(RA_ERR_SHAPE, "batch and seq_len must be >= 0, num_heads >= 1");
  if (!dtype_ok(d->a_dtype) || !dtype_ok(d->b_dtype) || !dtype_ok(d->out_dtype))
    return fail(RA_ERR_DTYPE, "unknown dtype");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  const int64_t strides[6] = {d->o_a_batch_stride,   d->o_b_batch_stride,   d->o_out_batch_stride,
                              d->lse_a_batch_stride, d->lse_b_batch_stride, d->lse_out_batch_stride};
  for (int i = 0; i < 6; ++i)
    if (strides[i] < 0) return fail(RA_ERR_SHAPE, "batch strides must be >= 0");
  const int64_t rows = (int64_t)d->seq_len * d->num_heads, elems = rows * d->head_dim;
  const int64_t oa_bs = pick(d->o_a_batch_stride, elems), ob_bs = pick(d->o_b_batch_stride, elems),
                oo_bs = pick(d->o_out_batch_stride, elems), la_bs = pick(d->lse_a_batch_stride, rows),
                lb_bs = pick(d->lse_b_batch_stride, rows), lo_bs = pick(d->lse_out_batch_stride, rows);
  if (d->batch > 1 && (oa_bs < elems || ob_bs < elems || oo_bs < elems || la_bs < rows ||
                       lb_bs < rows || lo_bs < rows))
    return fail(RA_ERR_SHAPE, "a batch stride is smaller than one batch row");
  if (d->batch == 0 || rows == 0) return RA_OK;
  if (!o_a || !o_b || !o_out || !lse_a || !lse_b || !lse_out)
    return fail(RA_ERR_NULL, "a merge operand is NULL");
  const size_t as = dtype_size(d->a_dtype), bs = dtype_size(d->b_dtype), os = dtype_size(d->out_dtype);
  const size_t need_a = as * 4, need_b = bs * 4, need_o = os * 4;  // 4-element vectors
  if (!aligned(o_a, need_a) || !aligned(o_b, need_b) || !aligned(o_out, need_o) ||
      (oa_bs * as) % need_a || (ob_bs * bs) % need_b || (oo_bs * os) % need_o)
    return fail(RA_ERR_ALIGN, "merge outputs/inputs must be aligned to 4 elements");
  if (!aligned(lse_a, 4) || !aligned(lse_b, 4) || !aligned(lse_out, 4))
    return fail(RA_ERR_ALIGN, "lse pointers must be 4-byte aligned");
  const size_t sa = span_bytes(d->batch, oa_bs, elems, as), sb = span_bytes(d->batch, ob_bs, elems, bs),
               so = span_bytes(d->batch, oo_bs, elems, os);
  const size_t la = span_bytes(d->batch, la_bs, rows, 4), lb = span_bytes(d->batch, lb_bs, rows, 4),
               lo = span_bytes(d->batch, lo_bs, rows, 4);
  auto same = [](const void *x, const void *y, int64_t xs, int64_t ys, int xd, int yd) {
    return x == y && xs == ys && xd == yd;
  };
  if (!same(o_out, o_a, oo_bs, oa_bs, d->out_dtype, d->a_dtype) && overlaps(o_out, so, o_a, sa))
    return fail(RA_ERR_ALIAS, "o_out overlaps o_a without being the same tensor");
  if (!same(o_out, o_b, oo_bs, ob_bs, d->out_dtype, d->b_dtype) && overlaps(o_out, so, o_b, sb))
    return fail(RA_ERR_ALIAS, "o_out overlaps o_b without being the same tensor");
  if (!same(lse_out, lse_a, lo_bs, la_bs, 0, 0) && overlaps(lse_out, lo, lse_a, la))
    return fail(RA_ERR_ALIAS, "lse_out overlaps lse_a without being the same tensor");
  if (!same(lse_out, lse_b, lo_bs, lb_bs, 0, 0) && overlaps(lse_out, lo, lse_b, lb))
    return fail(RA_ERR_ALIAS, "lse_out overlaps lse_b without being the same tensor");
  if (overlaps(lse_out, lo, o_out, so) || overlaps(lse_out, lo, o_a, sa) ||
      overlaps(lse_out, lo, o_b, sb) || overlaps(o_out, so, lse_a, la) || overlaps(o_out, so, lse_b, lb))
    return fail(RA_ERR_ALIAS, "an lse buffer overlaps an output buffer");
  ra::MergeParams p;
  p.oa = o_a;
  p.ob = o_b;
  p.la = lse_a;
  p.lb = lse_b;
  p.oo = o_out;
  p.lo = lse_out;
  p.oa_bs = oa_bs;
  p.ob_bs = ob_bs;
  p.oo_bs = oo_bs;
  p.la_bs = la_bs;
  p.lb_bs = lb_bs;
  p.lo_bs = lo_bs;
  p.batch = d->batch;
  p.seq = d->seq_len;
  p.heads = d->num_heads;
  p.d = d->head_dim;
  const hipError_t e = ra::launch_merge(p, d->a_dtype, d->b_dtype, d->out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge");
  return RA_OK;
}

}  // extern "C"

namespace {

// The backward's tile shapes: the dq pass uses the forward's (bm = 32 nt
// queries, bn = 64 keys); the dk/dv pass tiles keys by bwd_kv_tile(head_dim)
// and queries by kBwdQTile.
struct BwdShape {
  int32_t tnk, tnq, kvt;
};

ra_status check_bwd_desc(const ra_attn_desc *d, Resolved *r, BwdShape *bs) {
  ra_status st = check_desc(d, r);
  if (st != RA_OK) return st;
  if (r->split != 0) return fail(RA_ERR_UNSUPPORTED, "o_split_row applies to the forward's output only");
  if (d->qkv_dtype != RA_BF16)
    return fail(RA_ERR_UNSUPPORTED, "the backward needs bf16 q, k and v");
  // check_desc admits only the head-dim pairs the kernels have: equal, or MLA's 192 / 128
  const int kvt = ra::bwd_kv_tile(d->head_dim);
  const int64_t tnk = ((int64_t)d->kv_len + kvt - 1) / kvt;
  const int64_t tnq = ((int64_t)d->q_len + ra::kBwdQTile - 1) / ra::kBwdQTile;
  if (tnq > kMaxKeyTiles)
    return fail(RA_ERR_UNSUPPORTED, "q_len %d exceeds %lld query tiles of %d tokens", d->q_len,
                (long long)kMaxKeyTiles, ra::kBwdQTile);
  if ((int64_t)d->batch * d->num_kv_heads * tnk >= (int64_t)1 << 31)
    return fail(RA_ERR_UNSUPPORTED, "too many key tiles for one launch");
  bs->tnk = (int32_t)tnk;
  bs->tnq = (int32_t)tnq;
  bs->kvt = kvt;
  return RA_OK;
}

ra::BwdLayout bwd_layout_of(const ra_attn_desc *d, const Resolved &r, const BwdShape &bs) {
  return ra::bwd_workspace_layout(d->batch, d->q_len, d->num_q_heads, d->num_kv_heads,
                                  d->head_dim, r.dv, r.nqt, r.nkt, bs.tnq, bs.tnk);
}

// The mask with the roles of queries and keys swapped: with d = pos_q - pos_k
// the pair is visible iff lo <= d <= hi; seen from the key, -d must lie in
// [-hi, -lo], i.e. causal 0, left window -lo and right window hi.
ra::MaskParams swapped_mask(const ra_attn_desc *d) {
  ra::MaskParams m;
  m.causal = 0;
  m.wl = d->causal ? 0 : d->window_right;
  m.wr = d->window_left;
  return m;
}

}  // namespace

extern "C" {

ra_status ra_attn_bwd_workspace_size(const ra_attn_desc *desc, size_t *bytes) {
  Resolved r;
  BwdShape bs;
  const ra_status st = check_bwd_desc(desc, &r, &bs);
  if (st != RA_OK) return st;
  if (!bytes) return fail(RA_ERR_NULL, "bytes is NULL");
  *bytes = bwd_layout_of(desc, r, bs).total;
  return RA_OK;
}

ra_status ra_attn_bwd(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                      const int32_t *qid, const int32_t *qpos, const int32_t *kid,
                      const int32_t *kpos, const void *o, const float *lse, const void *dout,
                      int32_t grad_dtype, void *dq, void *dk, void *dv, void *workspace,
                      size_t workspace_bytes, ra_stream_t stream) {
  Resolved r;
  BwdShape bs;
  ra_status st = check_bwd_desc(d, &r, &bs);
  if (st != RA_OK) return st;
  if (!dtype_ok(grad_dtype)) return fail(RA_ERR_DTYPE, "unknown grad_dtype %d", grad_dtype);
  const bool has_q = d->batch > 0 && d->q_len > 0;
  const bool has_k = d->batch > 0 && d->kv_len > 0;
  if (has_q && (!q || !o || !lse || !dout || !dq)) return fail(RA_ERR_NULL, "q, o, lse, dout or dq is NULL");
  if (has_k && (!k || !v || !dk || !dv)) return fail(RA_ERR_NULL, "k, v, dk or dv is NULL");
  st = check_meta(d, r, qid, qpos, kid, kpos);
  if (st != RA_OK) return st;
  const size_t os = dtype_size(d->out_dtype), gs = dtype_size(grad_dtype);
  const void *p16[8] = {q, k, v, o, dout, dq, dk, dv};
  for (const void *ptr : p16)
    if (!aligned(ptr, 16)) return fail(RA_ERR_ALIGN, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  const int64_t sts[6] = {r.q_bs, r.kv_bs, r.q_ts, r.kv_ts, r.v_bs, r.v_ts};
  for (int i = 0; i < 6; ++i)
    if ((sts[i] * 2) % 16 || (sts[i] * (int64_t)gs) % 16)
      return fail(RA_ERR_ALIGN, "batch and token strides must be multiples of 16 bytes for every tensor using them");
  if ((r.o_bs * os) % 16 || (r.o_bs * 2) % 16 || (r.o_ts * os) % 16 || (r.o_ts * 2) % 16)
    return fail(RA_ERR_ALIGN, "batch and token strides must be multiples of 16 bytes for every tensor using them");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  const int64_t D = d->head_dim;
  const int64_t B = d->batch, Tq = d->q_len, Tk = d->kv_len;
  // row widths (elements): Q and K rows hold head_dim per head, V, O and dO
  // rows v_head_dim per head
  const int64_t Lq = (int64_t)d->num_q_heads * D, Lk = (int64_t)d->num_kv_heads * D;
  const int64_t Lo = (int64_t)d->num_q_heads * r.dv, Lv = (int64_t)d->num_kv_heads * r.dv;
  const size_t q_span = span_bytes2(B, Tq, Lq, r.q_bs, r.q_ts, 2);
  const size_t kv_span = span_bytes2(B, Tk, Lk, r.kv_bs, r.kv_ts, 2);
  const size_t v_span = span_bytes2(B, Tk, Lv, r.v_bs, r.v_ts, 2);
  const size_t o_span = span_bytes2(B, Tq, Lo, r.o_bs, r.o_ts, os);
  const size_t do_span = span_bytes2(B, Tq, Lo, r.o_bs, r.o_ts, 2);
  const size_t l_span = span_bytes(B, r.lse_bs, Tq * d->num_q_heads, 4);
  const size_t dq_span = span_bytes2(B, Tq, Lq, r.q_bs, r.q_ts, gs);
  const size_t dkv_span = span_bytes2(B, Tk, Lk, r.kv_bs, r.kv_ts, gs);
  const size_t dvv_span = span_bytes2(B, Tk, Lv, r.v_bs, r.v_ts, gs);
  const void *ins[6] = {q, k, v, o, lse, dout};
  const size_t in_span[6] = {q_span, kv_span, v_span, o_span, l_span, do_span};
  const void *outs[3] = {dq, dk, dv};
  const size_t out_span[3] = {dq_span, dkv_span, dvv_span};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_span[i], ins[j], in_span[j]))
        return fail(RA_ERR_ALIAS, "a gradient buffer overlaps an input");
  // The gradients may share one packed buffer (rows side by side at equal
  // strides, e.g. dk/dv of a packed K/V layout); otherwise their spans must not meet.
  const int64_t g = (int64_t)gs;
  const bool kv_same = r.kv_bs == r.v_bs && r.kv_ts == r.v_ts;
  if (kv_same ? rows_overlap(dk, Tk, Lk * g, dv, Tk, Lv * g, B, r.kv_bs * g, r.kv_ts * g)
              : overlaps(dk, dkv_span, dv, dvv_span))
    return fail(RA_ERR_ALIAS, "dk and dv overlap");
  const bool qk_same = r.q_bs == r.kv_bs && r.q_ts == r.kv_ts;
  const bool qv_same = r.q_bs == r.v_bs && r.q_ts == r.v_ts;
  if (qk_same ? rows_overlap(dq, Tq, Lq * g, dk, Tk, Lk * g, B, r.q_bs * g, r.q_ts * g)
              : overlaps(dq, dq_span, dk, dkv_span))
    return fail(RA_ERR_ALIAS, "dq overlaps dk");
  if (qv_same ? rows_overlap(dq, Tq, Lq * g, dv, Tk, Lv * g, B, r.q_bs * g, r.q_ts * g)
              : overlaps(dq, dq_span, dv, dvv_span))
    return fail(RA_ERR_ALIAS, "dq overlaps dv");
  const MetaSpans ms = meta_spans(d, r.qm_bs, r.km_bs, qid, qpos, kid, kpos);
  for (int i = 0; i < 3; ++i)
    if (overlaps_any(outs[i], out_span[i], ms.s, 4))
      return fail(RA_ERR_ALIAS, "a gradient buffer overlaps the segment ids or positions");
  if (!has_q && !has_k) return RA_OK;
  const ra::BwdLayout L = bwd_layout_of(d, r, bs);
  if (L.total > 0 && !workspace)
    return fail(RA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  {
    const Span used[13] = {{q, q_span},   {k, kv_span},   {v, v_span},     {o, o_span},
                           {lse, l_span}, {dout, do_span}, {dq, dq_span},  {dk, dkv_span},
                           {dv, dvv_span}, ms.s[0],        ms.s[1],        ms.s[2],
                           ms.s[3]};
    if (overlaps_any(workspace, L.total, used, 13))
      return fail(RA_ERR_ALIAS, "the workspace overlaps an input or output");
  }

  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  ra::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.qid = qid;
  p.qpos = qpos;
  p.kid = kid;
  p.kpos = kpos;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.lse2 = (float *)(ws + L.lse2);
  p.dsum = (float *)(ws + L.dsum);
  p.list = (const uint32_t *)(ws + L.list);
  p.count = (const int32_t *)(ws + L.count);
  p.tlist = (const uint32_t *)(ws + L.tlist);
  p.tcount = (const int32_t *)(ws + L.tcount);
  p.kvpack = ws + L.kvpack;
  p.qpack = ws + L.qpack;
  p.q_bs = r.q_bs;
  p.kv_bs = r.kv_bs;
  p.o_bs = r.o_bs;
  p.do_bs = r.o_bs;
  p.lse_bs = r.lse_bs;
  p.qm_bs = r.qm_bs;
  p.km_bs = r.km_bs;
  p.dq_bs = r.q_bs;
  p.dkv_bs = r.kv_bs;
  p.q_ts = r.q_ts;
  p.kv_ts = r.kv_ts;
  p.o_ts = r.o_ts;
  p.v_bs = r.v_bs;
  p.v_ts = r.v_ts;
  p.batch = d->batch;
  p.tq = d->q_len;
  p.tk = d->kv_len;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.nqt = r.nqt;
  p.nkt = r.nkt;
  p.tnk = bs.tnk;
  p.tnq = bs.tnq;
  p.scale = d->scale;
  p.scale_log2 = d->scale * 1.4426950408889634f;
  p.mask = mask_of(d);
  const bool out_bf16 = grad_dtype == RA_BF16;

  // Schedules: the forward's (query tiles x 64-key tiles) for dq, and the
  // swapped one (key tiles of bwd_kv_tile(head_dim) x 32-query tiles) for dk/dv.
  ra::Schedule fs;
  fs.qsum = (ra::TileSum *)(ws + L.qsum);
  fs.ksum = (ra::TileSum *)(ws + L.ksum);
  fs.count = (int32_t *)(ws + L.count);
  fs.pairs = (int64_t *)(ws + L.pairs);
  fs.list = (uint32_t *)(ws + L.list);
  ra::Schedule ts;
  ts.qsum = (ra::TileSum *)(ws + L.tqsum);
  ts.ksum = (ra::TileSum *)(ws + L.tksum);
  ts.count = (int32_t *)(ws + L.tcount);
  ts.pairs = (int64_t *)(ws + L.tpairs);
  ts.list = (uint32_t *)(ws + L.tlist);
  hipError_t e;
  if (has_q) {
    st = run_schedule(d, r, fs, qid, qpos, kid, kpos, nullptr, s);
    if (st != RA_OK) return st;
    e = ra::launch_bwd_prep(p, r.dv, d->out_dtype == RA_BF16, s);
    if (e != hipSuccess) return hip_fail(e, "backward prep");
  }
  if (has_k) {
    e = ra::launch_summaries(kid, kpos, r.km_bs, d->batch, d->kv_len, bs.kvt, bs.tnk, ts.qsum, s);
    if (e != hipSuccess) return hip_fail(e, "tile summaries (keys, swapped)");
    e = ra::launch_summaries(qid, qpos, r.qm_bs, d->batch, d->q_len, ra::kBwdQTile, bs.tnq, ts.ksum, s);
    if (e != hipSuccess) return hip_fail(e, "tile summaries (queries, swapped)");
    e = ra::launch_classify(ts, kid, kpos, qid, qpos, r.km_bs, r.qm_bs, d->batch, d->kv_len,
                            d->q_len, bs.kvt, ra::kBwdQTile, bs.tnk, bs.tnq,
                            swapped_mask(d), nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "tile classification (swapped)");
  }
  e = ra::launch_bwd_pack(p, d->head_dim, r.dv, s);
  if (e != hipSuccess) return hip_fail(e, "backward tile packing");
  if (has_q) {
    e = ra::launch_bwd_dq(p, d->head_dim, r.dv, r.nt, out_bf16, s);
    if (e != hipSuccess) return hip_fail(e, "backward dq pass");
  }
  if (has_k) {
    e = ra::launch_bwd_dkdv(p, d->head_dim, r.dv, out_bf16, s);
    if (e != hipSuccess) return hip_fail(e, "backward dk/dv pass");
  }
  return RA_OK;
}

static ra_status check_reorder(int32_t batch, int32_t seq, int64_t row_bytes, int32_t cp,
                               int32_t kind, int32_t stripe) {
  if (batch < 0 || seq < 0) return fail(RA_ERR_SHAPE, "batch and seq_len must be >= 0");
  if (row_bytes < 1) return fail(RA_ERR_SHAPE, "row_bytes must be >= 1");
  if (cp < 1) return fail(RA_ERR_SHAPE, "cp_size must be >= 1");
  if (kind == RA_REORDER_DUAL_CHUNK) {
    if (seq % (2 * cp)) return fail(RA_ERR_SHAPE, "dual chunk needs seq_len %% (2*cp_size) == 0");
  } else if (kind == RA_REORDER_STRIPED) {
    if (stripe < 1) return fail(RA_ERR_SHAPE, "stripe_size must be >= 1");
    if (seq % ((int64_t)cp * stripe))
      return fail(RA_ERR_SHAPE, "striped needs seq_len %% (cp_size*stripe_size) == 0");
  } else {
    return fail(RA_ERR_SHAPE, "unknown reorder kind %d", kind);
  }
  return RA_OK;
}

static ra_status do_reorder(const void *src, void *dst, int32_t batch, int32_t seq, int64_t row_bytes,
                            int32_t cp, int32_t kind, int32_t stripe, bool inverse,
                            ra_stream_t stream) {
  ra_status st = check_reorder(batch, seq, row_bytes, cp, kind, stripe);
  if (st != RA_OK) return st;
  if (batch == 0 || seq == 0) return RA_OK;
  if (!src || !dst) return fail(RA_ERR_NULL, "src or dst is NULL");
  const size_t bytes = (size_t)batch * seq * row_bytes;
  if (overlaps(src, bytes, dst, bytes)) return fail(RA_ERR_ALIAS, "src and dst overlap");
  const hipError_t e = ra::launch_reorder(src, dst, batch, seq, row_bytes, cp,
                                          kind == RA_REORDER_STRIPED ? 1 : 0, stripe, inverse,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reorder");
  return RA_OK;
}

ra_status ra_reorder(const void *src, void *dst, int32_t batch, int32_t seq_len, int64_t row_bytes,
                     int32_t cp_size, int32_t kind, int32_t stripe_size, ra_stream_t stream) {
  return do_reorder(src, dst, batch, seq_len, row_bytes, cp_size, kind, stripe_size, false, stream);
}

ra_status ra_inverse_reorder(const void *src, void *dst, int32_t batch, int32_t seq_len,
                             int64_t row_bytes, int32_t cp_size, int32_t kind, int32_t stripe_size,
                             ra_stream_t stream) {
  return do_reorder(src, dst, batch, seq_len, row_bytes, cp_size, kind, stripe_size, true, stream);
}

ra_status ra_reorder_index(int32_t seq_len, int32_t cp_size, int32_t kind, int32_t stripe_size,
                           int32_t inverse, int32_t *host_map) {
  ra_status st = check_reorder(1, seq_len, 1, cp_size, kind, stripe_size);
  if (st != RA_OK) return st;
  if (seq_len > 0 && !host_map) return fail(RA_ERR_NULL, "host_map is NULL");
  const int32_t k = kind == RA_REORDER_STRIPED ? 1 : 0;
  for (int64_t p = 0; p < seq_len; ++p)
    host_map[p] = (int32_t)(inverse ? ra::reorder_dst(p, seq_len, cp_size, k, stripe_size)
                                    : ra::reorder_src(p, seq_len, cp_size, k, stripe_size));
  return RA_OK;
}

}  // extern "C"
