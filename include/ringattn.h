/*
 * libringattn -- blockwise online-softmax attention forward for AMD MI355X (gfx950).
 *
 * Plain C ABI: device pointers and sizes in, status codes out.  No entry point
 * allocates device memory, synchronises the device, prints, throws or aborts.
 * Every argument is validated on the host before any HIP call; on a bad
 * argument the call returns a status, leaves all buffers untouched and records a
 * message for ra_last_error().  Kernel launches are enqueued on the caller's
 * stream (a hipStream_t; NULL is the default stream); faults inside a kernel
 * surface at the caller's next synchronisation.
 *
 * Tensor layouts ("THD": batch, tokens, heads, head_dim; head_dim contiguous):
 *   q  [B, Tq, Hq,  D]    k, v  [B, Tk, Hkv, D]    o  [B, Tq, Hq, D]
 *   lse [B, Tq, Hq] (fp32)   segment ids / positions [B, T] (int32)
 * Rows of one batch entry are contiguous; only the batch stride may differ from
 * the dense value, so sequence shards and ring chunks can be passed as views.
 *
 * Sources (web pages; sections named, no line numbers):
 *   [TUT] TransformerEngine JAX tutorial "JAX: Context-Parallel Attention with
 *         TransformerEngine": s1 packed THD inputs (segment ids / positions,
 *         padding id 0), s3 fused attention call (scaling_factor,
 *         PADDING_CAUSAL_MASK, window_size, THD_THD_THD, vanilla softmax),
 *         s4 striped load balancing (reorder_causal_load_balancing and its
 *         inverse, cp_size, seq_dim, stripe_size).
 *   [CPP] "Implementation: NVIDIA TransformerEngine JAX Cpp Attention":
 *         I/O contract (outputs: output, softmax_aux); FusedAttnHelper
 *         backend query.
 *   [RA]  "Context parallelism and ring attention": "The attention problem",
 *         "Ring attention", "Online softmax", "Causal attention", "Load balance".
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *ra_stream_t;
/* Same type as hipEvent_t. */
typedef struct ihipEvent_t *ra_event_t;

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  RA_ERR_SHAPE = 2,       /* a size, stride or window is out of range            */
  RA_ERR_DTYPE = 3,       /* unknown or unsupported dtype                        */
  RA_ERR_ALIGN = 4,       /* pointer or stride breaks the alignment rules        */
  RA_ERR_UNSUPPORTED = 5, /* valid request outside what the kernels implement    */
  RA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required             */
  RA_ERR_ALIAS = 7,       /* buffers overlap where they must not                 */
  RA_ERR_HIP = 8          /* a HIP call or launch failed (text in ra_last_error) */
} ra_status;

typedef enum ra_dtype { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

typedef enum ra_reorder_kind {
  RA_REORDER_DUAL_CHUNK = 0, /* 2R stripes; rank r holds stripe r, then stripe 2R-1-r ([RA] Load balance) */
  RA_REORDER_STRIPED = 1     /* stripes of stripe_size tokens; stripe j goes to rank j mod R ([TUT] s4)  */
} ra_reorder_kind;

/* Tile classes written by ra_classify_tiles ([RA] "Causal attention"). */
enum { RA_TILE_SKIP = 0, RA_TILE_PARTIAL = 1, RA_TILE_FULL = 2 };

/*
 * Attention problem description (the static configuration of one forward).
 *
 * Masking ([TUT] s1, s3): query i and key j of batch row b are visible to each
 * other iff  ids_q[i] != 0 && ids_q[i] == ids_kv[j]            (same segment, not padding)
 *        && (!causal || pos_kv[j] <= pos_q[i])                  (positions, never array indices)
 *        && (window_left  < 0 || pos_q[i] - pos_kv[j] <= window_left)
 *        && (window_right < 0 || pos_kv[j] - pos_q[i] <= window_right).
 * Query head h reads K/V head h / (Hq / Hkv).
 * Batch strides are in elements of the tensor they describe; 0 selects the dense
 * value (Tq * q token stride for q, and likewise for o, k and v; Tq*Hq for lse,
 * Tq / Tk for the int32 metadata).
 *
 * Layouts ([TUT] s1: separate-tensor THD and packed K/V THD_T2HD, BSHD; [CPP] the
 * qkv_layout field of the fused attention configuration): inside a
 * token the Hx*D values of q, k, v and o are contiguous (head, then head_dim),
 * but consecutive tokens may sit token_stride elements apart, so q, k, v may be
 * views into one packed tensor and the sequence may be the outer dimension:
 *   BSHD / THD with segment ids   token stride H*D, batch stride T*H*D (default)
 *   THD_T2HD (K/V packed)         k = kv, v = kv + Hkv*D, kv token stride 2*Hkv*D
 *   THD_T3HD (Q/K/V packed)       q = qkv, k = qkv + Hq*D, v = k + Hkv*D, all token
 *                                 strides (Hq + 2*Hkv)*D
 *   SBHD (sequence outermost)     token stride B*H*D, batch stride H*D
 * MLA head dimensions ([TUT] "Next steps", single-GPU attention): v and o may have their own
 * head dim Dv (v [B,Tk,Hkv,Dv], o [B,Tq,Hq,Dv]); the scale stays the caller's
 * (head_dim^-1/2 of q and k in [TUT] s3).  Supported (head_dim, Dv) pairs: (64, 64),
 * (128, 128) and, in bf16 (forward and backward), (192, 128).
 * The (batch, token) rows of each tensor must nest without overlap: with
 * L = H*D, either token stride >= L and batch stride >= (T-1)*token stride + L,
 * or batch stride >= L and token stride >= (B-1)*batch stride + L.
 *
 * Split output (ra_attn_fwd and ra_attn_fwd_accumulate only; every other entry
 * point requires o_split_row = 0): with 0 < o_split_row < Tq, query row t >=
 * o_split_row of batch row b is written at o + b*o_batch_stride +
 * t*o_token_stride + o_split_offset, and its LSE at lse + b*lse_batch_stride +
 * t*Hq + lse_split_offset.  A dual-chunk shard ([RA] "Load balance") is two
 * stripes of the sequence, so its result can go straight to the stripes'
 * original positions: the inverse reorder folded into the call.  Needs token
 * stride >= L; the offsets are >= 0, o_split_offset keeps o 16-byte aligned,
 * and with B > 1 each batch row's extent (gap included) fits in its batch
 * stride.  That extent must not overlap any input, and an accumulating call's
 * partial must then be a separate buffer (no in-place update).
 */
typedef struct ra_attn_desc {
  int32_t batch;          /* B  >= 0                                           */
  int32_t q_len;          /* Tq >= 0                                           */
  int32_t kv_len;         /* Tk >= 0                                           */
  int32_t num_q_heads;    /* Hq >= 1                                           */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0                           */
  int32_t head_dim;       /* D of q and k: 64, 128, or 192 with v_head_dim 128 */
  int32_t qkv_dtype;      /* ra_dtype of q, k and v                            */
  int32_t out_dtype;      /* ra_dtype of o                                     */
  float scale;            /* score scale, finite and > 0; head_dim^-1/2 in [TUT] s3 */
  int32_t causal;         /* 0 or 1                                            */
  int32_t window_left;    /* -1 (unbounded) or >= 0                            */
  int32_t window_right;   /* -1 (unbounded) or >= 0                            */
  int64_t q_batch_stride;
  int64_t kv_batch_stride;
  int64_t o_batch_stride;
  int64_t lse_batch_stride;
  int64_t q_meta_batch_stride;
  int64_t kv_meta_batch_stride;
  int64_t q_token_stride;   /* elements between consecutive tokens of q; 0 = Hq*D          */
  int64_t kv_token_stride;  /* the same for k and v (one value for both); 0 = Hkv*D         */
  int64_t o_token_stride;   /* the same for o (and a running partial, dout); 0 = Hq*Dv     */
  int32_t v_head_dim;       /* Dv, head dim of v and o; 0 = head_dim (see below)           */
  int32_t o_split_row;      /* 0, or a split row of the output (see below)                 */
  int64_t v_batch_stride;   /* v's strides; 0 = k's when Dv == head_dim, else dense        */
  int64_t v_token_stride;   /*   (Tk*Hkv*Dv and Hkv*Dv)                                    */
  int64_t o_split_offset;   /* elements: extra offset of o rows >= o_split_row (>= 0)      */
  int64_t lse_split_offset; /* elements: the same for lse (>= 0)                           */
} ra_attn_desc;

/* Library identification and diagnostics.  The returned strings are static
 * (ra_last_error: thread-local, valid until the thread's next failing call). */
const char *ra_version(void);
const char *ra_status_string(ra_status status);
const char *ra_last_error(void);

/*
 * Host-only support query (the role of FusedAttnHelper's backend query in
 * [CPP]): RA_OK if ra_attn_fwd implements this description, otherwise the
 * status it would return.  Supported: bf16 q/k/v (MFMA path) or fp32 q/k/v,
 * (head_dim, v_head_dim) of (64, 64) or (128, 128), and in bf16 also (192, 128),
 * bf16 or fp32 output, any Hq/Hkv group size, any lengths up to 2^21 key tokens
 * per call (2^20 for fp32).  Segment ids may be any int32 value (0 marks
 * padding; ids compare only within one batch row); positions must be
 * non-negative (the device does not check them).  Makes no HIP call.
 */
ra_status ra_check_support(const ra_attn_desc *desc);

/* Token tile sizes (query tile, key tile) that the forward and ra_classify_tiles
 * use for this description.  Host only. */
ra_status ra_tile_shape(const ra_attn_desc *desc, int32_t *bm_tokens, int32_t *bn_tokens);

/* Bytes of device workspace that ra_attn_fwd and ra_classify_tiles need for
 * this description (tile summaries and per-query-tile work lists).  Host only. */
ra_status ra_attn_fwd_workspace_size(const ra_attn_desc *desc, size_t *bytes);

/*
 * Exact masked softmax attention forward ([RA] "The attention problem";
 * [TUT] s3 fused_attn with PADDING_CAUSAL_MASK, window_size, no bias, no
 * dropout, vanilla softmax), evaluated blockwise over key tiles with the
 * online-softmax running max / sum / weighted sum ([RA] "Online softmax").
 * Key tiles with no visible pair are skipped, tiles that are all visible run
 * unmasked, and only the rest are masked ([RA] "Causal attention").
 *
 * Outputs ([CPP] I/O contract: output and softmax_aux):
 *   o   [B,Tq,Hq,D] out_dtype:  softmax(scale * q k^T + M) v
 *   lse [B,Tq,Hq]   fp32:       natural-log log-sum-exp of the visible scaled
 *                               scores; a query with no visible key gets
 *                               o = 0 and lse = -inf.
 * Both are fully overwritten.  q, k, v, o: 16-byte aligned, batch strides a
 * multiple of 16 bytes; metadata and lse 4-byte aligned.  o and lse must not
 * overlap q, k, v, the segment ids or positions, or each other.  workspace:
 * device memory of at least ra_attn_fwd_workspace_size() bytes, 256-byte
 * aligned, owned by the caller, overwritten, overlapping no other argument;
 * calls that share a workspace must be ordered on one stream.  Every overlap
 * named here is RA_ERR_ALIAS.
 */
ra_status ra_attn_fwd(const ra_attn_desc *desc, const void *q, const void *k, const void *v,
                      const int32_t *q_segment_ids, const int32_t *q_segment_pos,
                      const int32_t *kv_segment_ids, const int32_t *kv_segment_pos, void *o,
                      float *lse, void *workspace, size_t workspace_bytes, ra_stream_t stream);

/*
 * Accumulating forward: the same attention as ra_attn_fwd, merged in the
 * epilogue with a running partial result over other key sets ([RA] "Online
 * softmax": the ring's per-step update, fused into the step that produces the
 * new block):
 *   L = log(exp(LSE) + exp(partial.lse));  o = exp(LSE - L) O + exp(partial.lse - L) partial.o
 * where (O, LSE) is this call's attention; rows where either side is empty take
 * the other side unchanged (converted to out_dtype).  o/lse may be exactly
 * partial.o/partial.lse (same dtype and strides): the update is then in place
 * and query tiles with no visible pair in this call are not touched at all.
 * Any other overlap between o/lse and the partial is RA_ERR_ALIAS.  The partial
 * has o's shape [B,Tq,Hq,D] (dtype partial.dtype, 16-byte aligned) and lse's
 * shape [B,Tq,Hq] (fp32); its batch strides are in elements, 0 = dense.  All
 * other arguments, rules and the workspace are those of ra_attn_fwd.
 */
typedef struct ra_partial {
  const void *o;
  const float *lse;
  int32_t dtype; /* ra_dtype of o */
  int32_t reserved;
  int64_t o_batch_stride, lse_batch_stride;
} ra_partial;

ra_status ra_attn_fwd_accumulate(const ra_attn_desc *desc, const void *q, const void *k,
                                 const void *v, const int32_t *q_segment_ids,
                                 const int32_t *q_segment_pos, const int32_t *kv_segment_ids,
                                 const int32_t *kv_segment_pos, const ra_partial *partial, void *o,
                                 float *lse, void *workspace, size_t workspace_bytes,
                                 ra_stream_t stream);

/*
 * The forward with its per-call preparation split out, for repeated calls on
 * one segment layout (the ring driver's steps: several calls read each K/V
 * chunk, and the same calls recur every step).  The workspace of
 * ra_attn_fwd is two parts:
 *   schedule  the query/key tile summaries, the per-query-tile lists of key
 *             tiles to visit and their visible-pair counts: a function of the
 *             description (shapes, dtypes, head dims, mask) and of the four
 *             segment id / position tensors' values only;
 *   kv        the packed K/V tiles the bf16 kernel streams into LDS (with
 *             their ids and positions): a function of k, v, kv_segment_ids and
 *             kv_segment_pos only (empty for fp32 inputs).
 * ra_attn_fwd_workspace_parts gives the bytes of each (their sum is
 * ra_attn_fwd_workspace_size's, up to alignment).  ra_attn_fwd_ex is
 * ra_attn_fwd (partial == NULL) or ra_attn_fwd_accumulate (partial != NULL)
 * with the two parts in separate caller-owned buffers (256-byte aligned, not
 * overlapping each other or any argument).  Without flags it writes both
 * parts, then runs the attention; with RA_FWD_SCHEDULE_READY it skips the
 * classification and reads schedule_ws as written by an earlier call with an
 * equal description and equal segment id / position values; with
 * RA_FWD_KV_READY it skips the packing and reads kv_ws as written by an
 * earlier call with equal k, v, kv_segment_ids and kv_segment_pos values and
 * equal shapes.  The library cannot check those two promises: a flag set on
 * a buffer that holds anything else gives wrong results (the kernels clamp
 * what they read from the schedule to the call's tile ranges, so they never
 * read outside the buffers).  Results are bit-identical to ra_attn_fwd /
 * ra_attn_fwd_accumulate.  Unknown flag bits are RA_ERR_SHAPE.
 */
#define RA_FWD_SCHEDULE_READY 1u
#define RA_FWD_KV_READY 2u

ra_status ra_attn_fwd_workspace_parts(const ra_attn_desc *desc, size_t *schedule_bytes,
                                      size_t *kv_bytes);

ra_status ra_attn_fwd_ex(const ra_attn_desc *desc, const void *q, const void *k, const void *v,
                         const int32_t *q_segment_ids, const int32_t *q_segment_pos,
                         const int32_t *kv_segment_ids, const int32_t *kv_segment_pos,
                         const ra_partial *partial, void *o, float *lse, void *schedule_ws,
                         size_t schedule_bytes, void *kv_ws, size_t kv_bytes, uint32_t flags,
                         ra_stream_t stream);

/*
 * The forward of ra_attn_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc.  Same arguments, rules and results as ra_attn_fwd
 * (bit-identical outputs), but no workspace argument: the tile lists and the
 * packed K/V tiles go to a scratch buffer of RA_NOALLOC_SCRATCH_BYTES that
 * the library holds as a static device array, one per GPU, reserved when the
 * library is loaded onto that GPU and kept until the process ends.  The call
 * allocates nothing and uses the current device's scratch (the stream must
 * belong to the current device).  A description whose
 * ra_attn_fwd_workspace_size() exceeds RA_NOALLOC_SCRATCH_BYTES is refused
 * with RA_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares
 * that GPU's scratch: calls that may overlap in time on one GPU (different
 * streams, or threads without ordering) race and must not be made; calls
 * ordered on one stream are safe.  Nothing in the scratch needs to start at
 * zero: each call writes all it reads.
 */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

ra_status ra_attn_fwd_noalloc(const ra_attn_desc *desc, const void *q, const void *k,
                              const void *v, const int32_t *q_segment_ids,
                              const int32_t *q_segment_pos, const int32_t *kv_segment_ids,
                              const int32_t *kv_segment_pos, void *o, float *lse,
                              ra_stream_t stream);

/*
 * Measurement hook (for timing the attention kernel apart from the tile
 * classification and K/V packing that precede it in the same call).  The next
 * ra_attn_fwd or ra_attn_fwd_accumulate call made on the calling thread
 * records `start` on its stream immediately before its attention kernel and
 * `stop` immediately after it.  Both are events the caller created
 * (hipEventCreate) and keeps owning; both NULL disarms a pending pair, exactly
 * one NULL is RA_ERR_NULL.  The pair is consumed by that one call: a call that
 * fails, or that launches no attention kernel (an empty batch), leaves the
 * events unrecorded.  Records only; it never synchronises.
 */
ra_status ra_profile_next_kernel(ra_event_t start, ra_event_t stop);

/*
 * The exact tile classes of the mask at the tile shape of ra_tile_shape()
 * ([RA] "Causal attention": skip / full / partial), and the number of visible
 * (query, key) pairs of every batch row.  classes: int8 [B, ceil(Tq/bm),
 * ceil(Tk/bn)] with RA_TILE_* values (a tile's class is decided over its
 * in-range pairs only); visible_pairs: int64 [B].  Either output may be NULL.
 * Only the metadata fields of desc matter (dtypes and head_dim select the tile
 * shape).  Same workspace rules as ra_attn_fwd; classes and visible_pairs
 * must not overlap the metadata, the workspace or each other (RA_ERR_ALIAS).
 */
ra_status ra_classify_tiles(const ra_attn_desc *desc, const int32_t *q_segment_ids,
                            const int32_t *q_segment_pos, const int32_t *kv_segment_ids,
                            const int32_t *kv_segment_pos, int8_t *classes,
                            int64_t *visible_pairs, void *workspace, size_t workspace_bytes,
                            ra_stream_t stream);

/*
 * Merge of two partial results over disjoint key sets ([RA] "Online softmax",
 * written over (output, log-sum-exp) pairs):
 *   lse = log(exp(lse_a) + exp(lse_b));  o = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b.
 * A row whose two inputs are both -inf gets o = 0, lse = -inf; a row with one
 * -inf input gets the other input unchanged (converted to out_dtype).  Never NaN
 * for finite inputs.  o_out may be exactly o_a or o_b (same dtype and strides;
 * lse likewise) for in-place accumulation; any other overlap is RA_ERR_ALIAS.
 * o_*: 16-byte aligned (8 for bf16 with D=64 strides), batch strides in
 * elements (0 = dense seq_len*num_heads*head_dim; lse: seq_len*num_heads).
 */
typedef struct ra_merge_desc {
  int32_t batch, seq_len, num_heads, head_dim; /* head_dim: 64 or 128        */
  int32_t a_dtype, b_dtype, out_dtype;         /* ra_dtype of o_a, o_b, o_out */
  int64_t o_a_batch_stride, o_b_batch_stride, o_out_batch_stride;
  int64_t lse_a_batch_stride, lse_b_batch_stride, lse_out_batch_stride;
} ra_merge_desc;

ra_status ra_attn_merge(const ra_merge_desc *desc, const void *o_a, const float *lse_a,
                        const void *o_b, const float *lse_b, void *o_out, float *lse_out,
                        ra_stream_t stream);

/*
 * Attention backward: the gradients of ra_attn_fwd's o with respect to q, k and
 * v, given the output gradient dout ([RA] "The attention problem" for the
 * function differentiated; [TUT] s5 times the forward together with this
 * backward, and [CPP] lists the backward primitives beside the forward ones).
 * Per query head h reading K/V head g = h / (Hq/Hkv), with the forward's lse:
 *   P  = exp(scale * q_h k_g^T + M - lse)        (0 where M masks; rows without
 *                                                  a visible key are all 0)
 *   dS = P * (dout_h v_g^T - rowsum(dout_h * o_h))
 *   dq_h = scale * dS k_g,   dk_g = scale * sum_h dS^T q_h,   dv_g = sum_h P^T dout_h
 * The mask M and every other rule of desc are ra_attn_fwd's; o and lse must be
 * that forward's outputs for the same inputs (P is rebuilt from lse; no max or
 * sum is recomputed).  Key tiles with no visible pair are skipped and only
 * boundary tiles are masked, in both passes: dq over the forward's tile lists,
 * dk/dv over lists built with the roles of keys and queries swapped.
 *
 * Inputs:  q, k, v bf16 (qkv_dtype must be RA_BF16); o [B,Tq,Hq,Dv] out_dtype
 *          with o_batch_stride; lse [B,Tq,Hq] fp32 with lse_batch_stride;
 *          dout [B,Tq,Hq,Dv] bf16 with o_batch_stride (in its own elements).
 * Outputs: dq like q (q_batch_stride), dk like k (kv_batch_stride), dv like v
 *          (v's strides, [B,Tk,Hkv,Dv]), all
 *          of dtype grad_dtype (RA_BF16 or RA_F32), fully overwritten: rows no
 *          visible pair reaches (padding, masked keys) get 0.  Each key's
 *          dk/dv is accumulated in registers over its whole query-head group
 *          and written once: no atomics, and the result does not depend on
 *          scheduling.
 * q, k, v, o, dout, dq, dk, dv: 16-byte aligned, batch strides multiples of 16
 * bytes; lse and metadata 4-byte aligned.  dq, dk and dv must not overlap each
 * other or any input, metadata included, and the workspace must overlap no
 * argument (RA_ERR_ALIAS).  workspace: device memory of at least
 * ra_attn_bwd_workspace_size() bytes, 256-byte aligned, owned by the caller,
 * overwritten (both passes' tile lists, rowsum(dout*o), and packed copies of
 * q/dout and k/v tiles in the layouts the kernels read); calls that share a
 * workspace must be ordered on one stream.  Supported: (head_dim, Dv) of
 * (64, 64), (128, 128) or MLA's (192, 128), any GQA group, Tq up to 2^20 and
 * Tk up to 2^21 tokens per call.
 */
ra_status ra_attn_bwd_workspace_size(const ra_attn_desc *desc, size_t *bytes);

ra_status ra_attn_bwd(const ra_attn_desc *desc, const void *q, const void *k, const void *v,
                      const int32_t *q_segment_ids, const int32_t *q_segment_pos,
                      const int32_t *kv_segment_ids, const int32_t *kv_segment_pos,
                      const void *o, const float *lse, const void *dout, int32_t grad_dtype,
                      void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                      ra_stream_t stream);

/*
 * Causal load-balancing permutation of the sequence axis of a dense
 * [batch, seq_len, row_bytes] tensor (any of q, k, v, segment ids/positions, o,
 * lse) -- [TUT] s4 reorder_causal_load_balancing with seq_dim 1:
 *   ra_reorder:          dst[b, p] = src[b, map(p)]
 *   ra_inverse_reorder:  dst[b, map(p)] = src[b, p]
 * where map is RA_REORDER_DUAL_CHUNK (needs seq_len % (2*cp_size) == 0) or
 * RA_REORDER_STRIPED (needs seq_len % (cp_size*stripe_size) == 0).  After a
 * reorder, rank r's shard is the contiguous token range [r*T/R, (r+1)*T/R).
 * src and dst must not overlap.  Rows are copied as bytes (row_bytes >= 1).
 */
ra_status ra_reorder(const void *src, void *dst, int32_t batch, int32_t seq_len, int64_t row_bytes,
                     int32_t cp_size, int32_t kind, int32_t stripe_size, ra_stream_t stream);
ra_status ra_inverse_reorder(const void *src, void *dst, int32_t batch, int32_t seq_len,
                             int64_t row_bytes, int32_t cp_size, int32_t kind, int32_t stripe_size,
                             ra_stream_t stream);

/* Host-side copy of the same map (host_map[p] = map(p), or its inverse when
 * inverse != 0), computed by the function the kernels use.  host_map: int32 [seq_len]. */
ra_status ra_reorder_index(int32_t seq_len, int32_t cp_size, int32_t kind, int32_t stripe_size,
                           int32_t inverse, int32_t *host_map);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
