// Internal interface between the C-ABI front end (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ringattn.h"

namespace ra {

// Token tiles.  The bf16 MFMA forward works on query tiles of 32*NT tokens
// (NT token sub-tiles of 32 per workgroup, 8/NT heads) and key tiles of 64;
// the fp32 forward on 64 x 32.
constexpr int kBnBf16 = 64;
constexpr int kBnF32 = 32;
constexpr int kBmF32 = 64;
constexpr int kWaves = 8;  // waves per bf16 workgroup

// Per-tile summary of a run of tokens (over valid, in-range tokens).
struct TileSum {
  int32_t nvalid;  // tokens with id != 0
  int32_t ninr;    // in-range tokens
  int32_t idmin, idmax;
  int32_t posmin, posmax;
  int32_t pad0, pad1;
};

struct MaskParams {
  int32_t causal;
  int32_t wl, wr;
};

struct Schedule {
  TileSum *qsum;      // [B, nqt]
  TileSum *ksum;      // [B, nkt]
  int32_t *count;     // [B, nqt] non-skip key tiles per query tile
  int64_t *pairs;     // [B, nqt] visible pairs per query tile
  uint32_t *list;     // [B, nqt, nkt] key tile | 0x80000000 if partial
};

struct WorkspaceLayout {
  size_t qsum, ksum, count, pairs, list, kpack, vpack, mpack, total;
};

// packed_head_dim > 0 adds room for the packed K / V^T / metadata tiles of the
// bf16 forward (batch * hkv * nkt tiles); packed_v_dim is V's head dim.
WorkspaceLayout workspace_layout(int32_t batch, int32_t nqt, int32_t nkt, int32_t hkv = 0,
                                 int32_t packed_head_dim = 0, int32_t packed_v_dim = 0);
// Bytes of one packed 64-key K block for a Q/K head dim (rows padded for 192).
size_t packed_k_block_bytes(int32_t head_dim);

// Packed K/V tiles of the bf16 forward.
struct PackParams {
  const void *k, *v;
  const int32_t *kid, *kpos;
  void *kpack, *vpack;
  int32_t *mpack;
  int64_t kv_bs, km_bs;
  int64_t kv_ts;             // token stride of K (elements)
  int64_t v_bs, v_ts;        // batch and token strides of V
  int32_t batch, tk, hkv, nkt;
};
hipError_t launch_pack_kv(const PackParams &p, int32_t head_dim, int32_t v_head_dim,
                          hipStream_t stream);

struct AttnParams {
  const void *q, *k, *v;
  const int32_t *qid, *qpos, *kid, *kpos;
  void *o;
  float *lse;
  const uint32_t *list;
  const int32_t *count;
  const void *kpack, *vpack;   // bf16 path: packed tiles written by pack_kv
  const int32_t *mpack;
  int64_t q_bs, kv_bs, o_bs, lse_bs, qm_bs, km_bs;  // batch strides (elements)
  int64_t q_ts, kv_ts, o_ts;  // token strides (elements); the running partial has o's
  int64_t v_bs, v_ts;         // V's batch and token strides
  int32_t batch, tq, tk, hq, hkv, group;
  int32_t nqt, nkt;
  float scale;       // score scale
  float scale_log2;  // scale * log2(e)
  MaskParams mask;
  // Optional running partial merged into the result in the epilogue.
  const void *acc_o;
  const float *acc_lse;
  int64_t acc_o_bs, acc_lse_bs;
  int32_t acc_mode;      // 0 none, 1 fp32 partial, 2 bf16 partial
  int32_t acc_in_place;  // o/lse are the partial itself: untouched tiles are skipped
  // Split output: query rows >= o_split (INT32_MAX: none) are written
  // o_split_off / lse_split_off elements further on in o / lse.
  int32_t o_split;
  int64_t o_split_off, lse_split_off;
};

// Launchers (return the launch's hipError_t).
hipError_t launch_summaries(const int32_t *ids, const int32_t *pos, int64_t meta_bs, int32_t batch,
                            int32_t len, int32_t tile, int32_t ntiles, TileSum *out,
                            hipStream_t stream);
hipError_t launch_classify(const Schedule &s, const int32_t *qid, const int32_t *qpos,
                           const int32_t *kid, const int32_t *kpos, int64_t qm_bs, int64_t km_bs,
                           int32_t batch, int32_t tq, int32_t tk, int32_t bm, int32_t bn,
                           int32_t nqt, int32_t nkt, MaskParams mask, int8_t *classes,
                           hipStream_t stream);
hipError_t launch_pair_sums(const int64_t *pairs, int32_t batch, int32_t nqt, int64_t *out,
                            hipStream_t stream);
// bf16 MFMA forward; nt = token sub-tiles per workgroup (1, 2, 4 or 8).
hipError_t launch_attn_bf16(const AttnParams &p, int32_t head_dim, int32_t v_head_dim, int32_t nt,
                            bool out_bf16, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams &p, int32_t head_dim, bool out_bf16,
                           hipStream_t stream);

struct MergeParams {
  const void *oa, *ob;
  const float *la, *lb;
  void *oo;
  float *lo;
  int64_t oa_bs, ob_bs, oo_bs, la_bs, lb_bs, lo_bs;
  int32_t batch, seq, heads, d;
};
hipError_t launch_merge(const MergeParams &p, int32_t a_dtype, int32_t b_dtype, int32_t out_dtype,
                        hipStream_t stream);

hipError_t launch_reorder(const void *src, void *dst, int32_t batch, int32_t seq, int64_t row_bytes,
                          int32_t cp, int32_t kind, int32_t stripe, bool inverse,
                          hipStream_t stream);

// ----------------------------------------------------------------------------- backward

constexpr int kBwdQTile = 32;    // queries per packed tile of the dK/dV pass
// dK/dV workgroup: waves of 32 keys each; 8 (two per SIMD) for head dims up
// to 128, 4 (one per SIMD, whose registers hold the 192-wide K rows and both
// accumulators) for the MLA head dims.
constexpr int bwd_kv_waves(int d) { return d == 192 ? 4 : 8; }
constexpr int bwd_kv_tile(int d) { return 32 * bwd_kv_waves(d); }

// Bytes of one packed K/V tile of the dQ pass (K, V and K^T blocks, ids and
// positions) and of one packed Q/dO tile of the dK/dV pass (Q and dO rows,
// then LSE*log2(e), rowsum(dO*O), ids and positions).  d is the head dim of Q
// and K, dv that of V, O and dO.  K/V rows carry 8 elements of padding; a Q or
// dO row of width w is bwd_qrow(w) elements long (see there).
constexpr size_t bwd_kv_tile_bytes(int d, int dv) {
  return (size_t)kBnBf16 * (d + 8) * 2 + (size_t)kBnBf16 * (dv + 8) * 2 +
         (size_t)d * (kBnBf16 + 8) * 2 + 2 * kBnBf16 * 4;
}
// Row length of the packed Q and dO blocks: 8 elements of padding.  The dK/dV
// pass reads them two ways: 16-byte pieces of 16 rows (row-major operands) and,
// with the LDS transpose load, 8-byte pieces of 4 rows, 32 lanes of which (two
// neighbouring 32-byte column pieces of the same 4 rows) are served together.
// Over 64 four-byte banks the first is free of conflicts when the 16 rows start
// 4 words apart modulo 64, the second when the 4 rows start 16 words apart.
// Rows of w + 8 elements (68, 36 or 100 words for w = 128, 64, 192) pass the
// first for any 16 consecutive rows and the second for rows 4 apart, which is
// the order in which the pass takes the queries of a tile (bwd_qperm).
constexpr int bwd_qrow(int w) { return w + 8; }
constexpr size_t bwd_q_tile_bytes(int d, int dv) {
  return (size_t)kBwdQTile * bwd_qrow(d) * 2 + (size_t)kBwdQTile * bwd_qrow(dv) * 2 +
         4 * kBwdQTile * 4;
}

struct BwdLayout {
  size_t qsum, ksum, count, pairs, list;        // dQ schedule (forward tile shape)
  size_t tqsum, tksum, tcount, tpairs, tlist;   // dK/dV schedule (key tiles x query tiles)
  size_t lse2, dsum, kvpack, qpack, total;
};
BwdLayout bwd_workspace_layout(int32_t batch, int32_t tq, int32_t hq, int32_t hkv, int32_t d,
                               int32_t dv, int32_t nqt, int32_t nkt, int32_t tnq, int32_t tnk);

struct BwdParams {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  const int32_t *qid, *qpos, *kid, *kpos;
  void *dq, *dk, *dv;
  float *lse2, *dsum;                  // [B, Tq, Hq], dense
  const uint32_t *list;                // dQ pass: per query tile, key tiles (| partial bit)
  const int32_t *count;
  const uint32_t *tlist;               // dK/dV pass: per key tile, 32-query tiles
  const int32_t *tcount;
  void *kvpack, *qpack;
  int64_t q_bs, kv_bs, o_bs, do_bs, lse_bs, qm_bs, km_bs, dq_bs, dkv_bs;
  int64_t q_ts, kv_ts, o_ts;           // token strides: dq like q, dk like k, dO like o
  int64_t v_bs, v_ts;                  // V's strides, also dv's
  int32_t batch, tq, tk, hq, hkv, group;
  int32_t nqt, nkt;                    // dQ schedule tiles
  int32_t tnk, tnq;                    // dK/dV schedule: key tiles, 32-query tiles
  float scale, scale_log2;
  MaskParams mask;
};
// rowsum(dO * O) and LSE * log2(e) (+inf for a row without visible key);
// v_head_dim is the width of O and dO.
hipError_t launch_bwd_prep(const BwdParams &p, int32_t v_head_dim, bool o_bf16,
                           hipStream_t stream);
// Packed tiles of both passes.
hipError_t launch_bwd_pack(const BwdParams &p, int32_t head_dim, int32_t v_head_dim,
                           hipStream_t stream);
// dQ pass (workgroups shaped like the forward's: nt token sub-tiles) and dK/dV pass.
hipError_t launch_bwd_dq(const BwdParams &p, int32_t head_dim, int32_t v_head_dim, int32_t nt,
                         bool out_bf16, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams &p, int32_t head_dim, int32_t v_head_dim,
                           bool out_bf16, hipStream_t stream);

// Heads per bf16 workgroup for a GQA group size, and the token sub-tiles.
inline int32_t bf16_heads_per_wg(int32_t group) {
  int32_t nh = 8;
  while (nh > 1 && group % nh) nh >>= 1;
  return nh;
}
inline int32_t bf16_token_subtiles(int32_t group) { return kWaves / bf16_heads_per_wg(group); }

}  // namespace ra
