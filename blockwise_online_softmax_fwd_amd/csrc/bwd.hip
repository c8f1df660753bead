// Attention backward for bf16 Q/K/V/dO on gfx950 matrix cores.
//
// Gradients of O = softmax(scale * Q K^T + M) V ("Context parallelism and ring
// attention", "The attention problem"; the TransformerEngine JAX tutorial
// times this backward together with the forward, section 5).  Per query head
// h reading K/V head g, with P = exp(scale * Q K^T + M - LSE) recomputed from
// the forward's LSE (no max, no sum):
//   dV_g += P^T dO,   dP = dO V^T,   dS = P * (dP - D)  with D = rowsum(dO * O),
//   dQ = scale * dS K,   dK_g += scale * dS^T Q.
//
// Kernels:
//  * prep: D and LSE * log2(e) for every (b, t, h) row (+inf where the row saw
//    no key, so its probabilities come out 0 without special cases).
//  * pack: per 64-key tile of one K/V head, K and V as [key][d] and K^T as
//    [d][key] (the dQ pass); per 32-query tile of one query head, Q and dO as
//    [query][d], LSE*log2(e), D, ids and positions (the dK/dV pass, which
//    reads the transposes of Q and dO from those rows with the LDS transpose
//    load, and takes a tile's queries in the order bwd_qperm, in which the
//    per-query values are stored).  Rows are padded instead of swizzled: 16 lanes reading the same
//    16-byte column of 16 consecutive rows then hit distinct LDS banks, and
//    each lane's operand addresses differ by constants only (one address
//    register per block instead of one per swizzled chunk).  The K^T block
//    uses the forward's token order inside 16-token chunks (vt_key).
//  * dQ pass: the forward's workgroup shape and work lists.  Per key tile a
//    wave forms S^T = K Q^T and dP^T = V dO^T, then dS^T, and accumulates
//    dQ^T += K^T dS^T; S and dP never leave registers.
//  * dK/dV pass: 8 waves, two per SIMD, each owning 32 keys of one K/V head
//    (their K and V are the B operands, held in registers).  The work list of
//    the 256-key tile (from the same classification kernels run with keys and
//    queries swapped) names the 32-query tiles that see it; every one of them
//    is visited once per query head of the group (head by head), so the
//    group's sum lands in registers and each key's gradients are written once,
//    without atomics.
//    Per visit: S = Q K^T and dP = dO V^T (lane = key, rows = queries), then
//    dV^T += dO^T P and dK^T += Q^T dS.
// D is the head dim of Q and K, DV that of V, O and dO (equal, or the MLA pair
// 192 / 128, for which the dK/dV workgroup has 4 waves: one per SIMD, whose
// registers then hold the 192-wide K rows and both accumulators).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stddef.h>

#include "bf16_tiles.h"
#include "internal.h"
#include "xcd_order.h"

namespace ra {
namespace {

using namespace tiles;

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16-byte MFMA operand taken across the rows of a row-major LDS block (row
// stride R elements) with the LDS transpose load, which, in each group of 16
// lanes, gives lane i the 16-bit element i % 4 of the 8-byte reads of lanes
// 4j + i / 4, j = 0..3.  When lane 4j + s of the group reads columns
// c0 + 4s .. c0 + 4s + 3 of row r_j, lane i receives column c0 + i of rows
// r_0 .. r_3; the second load, 2 rows further on, gives rows r_j + 2.
//
// The block is published by an explicit wait for the tile loads and a
// barrier.  The compiler would also wait for every LDS DMA still in flight
// (the next tile's, into another buffer) before a transpose load; through a
// restrict pointer it does not.
__device__ __forceinline__ bf16x8 tr_operand(const bf16 *__restrict__ lanep, int R) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lanep));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lanep + 2 * R));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Query order of the dK/dV pass inside a 32-query tile.  Row i of the score
// accumulator (A-operand lane i, i = 16c + 8b + 4h + j) holds query
// 16c + 4j + 2b + h of the tile.  The transposed operands of step c, half h,
// then take rows 4j + (const) of the packed block, 4 rows apart, and the
// row-major operands of lanes 0..15 (or 16..31) still take 16 distinct rows of
// one 16-row half; both read patterns are then free of bank conflicts with
// rows of w + 8 elements.  The packed tile keeps Q and dO in token order and
// stores its per-query values (LSE, D, ids, positions) in this order.
__host__ __device__ constexpr int bwd_qperm(int i) {
  return (i & 16) | ((i & 3) << 2) | (((i >> 3) & 1) << 1) | ((i >> 2) & 1);
}

constexpr int BN = kBnBf16;      // keys per tile of the dQ pass
constexpr int BQ = kBwdQTile;    // queries per tile of the dK/dV pass
constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------------------- prep

// DV: head dim of O and dO.  Token by token: the hq rows of a token are
// contiguous, so a row's index needs no division; several rows per thread
// are in flight at once.
template <int DV, bool OBF>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int TPR = DV / 4;      // threads per row, 4 elements each
  constexpr int RPB = 256 / TPR;   // rows per block and step
  constexpr int UN = 8;            // steps whose loads are issued together
  const int64_t tokens = (int64_t)p.batch * p.tq;
  const int sub = threadIdx.x % TPR;
  const int hq = p.hq;
  for (int64_t tok = blockIdx.x; tok < tokens; tok += gridDim.x) {
    const int64_t b = tok / p.tq, t = tok - b * p.tq;
    const bf16 *dob = (const bf16 *)p.dout + b * p.do_bs + t * p.o_ts + sub * 4;
    const int64_t ooff = b * p.o_bs + t * p.o_ts + sub * 4;
    for (int h0 = threadIdx.x / TPR; h0 < hq; h0 += RPB * UN) {
      float dot[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int h = h0 + u * RPB;
        dot[u] = 0.0f;
        if (h < hq) {
          const bf16x4 dov = *(const bf16x4 *)(dob + (int64_t)h * DV);
          if (OBF) {
            const bf16x4 ov = *(const bf16x4 *)((const bf16 *)p.o + ooff + (int64_t)h * DV);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot[u] = fmaf((float)dov[e], (float)ov[e], dot[u]);
          } else {
            const f32x4 ov = *(const f32x4 *)((const float *)p.o + ooff + (int64_t)h * DV);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot[u] = fmaf((float)dov[e], ov[e], dot[u]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int h = h0 + u * RPB;   // the same for the TPR lanes of a row
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) dot[u] += __shfl_xor(dot[u], off, TPR);
        if (sub == 0 && h < hq) {
          const int64_t r = tok * hq + h;
          const float l = p.lse[b * p.lse_bs + t * hq + h];
          p.dsum[r] = dot[u];
          p.lse2[r] = l == -INFINITY ? INFINITY : l * kLog2e;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- packing

// Row strides (elements) of the padded blocks.
template <int D> constexpr int kRowN = D + 8;        // [token][d] rows
constexpr int kRowTK = BN + 8;                       // K^T rows (64 keys)

template <int D, int DV>
struct KvTile {                 // one packed tile of the dQ pass
  bf16 k[BN * kRowN<D>];        // [key][d]
  bf16 v[BN * kRowN<DV>];       // [key][d]
  bf16 kt[D * kRowTK];          // [d][key], token order vt_key
  int32_t meta[2 * BN];         // ids, positions (0 past the end)
};

template <int D, int DV>
struct QTile {                  // one packed tile of the dK/dV pass
  bf16 qn[BQ * bwd_qrow(D)];    // [query][d]; the transposed operands are read
  bf16 don[BQ * bwd_qrow(DV)];  // from these rows with the LDS transpose load
  float lse2[BQ];               // LSE * log2(e); +inf past the end or for a row without keys
  float dsum[BQ];               // rowsum(dO * O)
  int32_t qid[BQ];
  int32_t qpos[BQ];
};

template <int D, int DV>
__global__ __launch_bounds__(256) void bwd_pack_kv_kernel(BwdParams p) {
  constexpr int KC = D / 8;              // 16-byte chunks of data per [key][d] row of K
  constexpr int VC = DV / 8;             // ... of V
  constexpr int RN = kRowN<D> / 8;       // chunks per padded row of K
  constexpr int RNV = kRowN<DV> / 8;     // ... of V
  constexpr int RT = kRowTK / 8;
  static_assert(sizeof(KvTile<D, DV>) == bwd_kv_tile_bytes(D, DV), "packed K/V tile size");
  __shared__ __attribute__((aligned(16))) bf16 ks[BN][D + 8];
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t tile = ((int64_t)b * p.hkv + g) * p.nkt + kt;
  KvTile<D, DV> *out = (KvTile<D, DV> *)((char *)p.kvpack + tile * sizeof(KvTile<D, DV>));
  const bf16 *kb = (const bf16 *)p.k + b * p.kv_bs + (int64_t)g * D;
  const bf16 *vb = (const bf16 *)p.v + b * p.v_bs + (int64_t)g * DV;
  const int64_t tok = p.kv_ts;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int u = tid; u < BN * RN; u += 256) {
    const int r = u / RN, c = u % RN;
    const int key = kt * BN + r;
    const bool in = key < p.tk && c < KC;
    const u32x4 kv = in ? *(const u32x4 *)(kb + key * tok + c * 8) : zero;
    *(u32x4 *)(out->k + u * 8) = kv;
    if (c < KC) *(u32x4 *)&ks[r][c * 8] = kv;
  }
  for (int u = tid; u < BN * RNV; u += 256) {
    const int r = u / RNV, c = u % RNV;
    const int key = kt * BN + r;
    const bool in = key < p.tk && c < VC;
    *(u32x4 *)(out->v + u * 8) = in ? *(const u32x4 *)(vb + key * p.v_ts + c * 8) : zero;
  }
  if (tid < BN) {
    const int key = kt * BN + tid;
    out->meta[tid] = key < p.tk ? p.kid[b * p.km_bs + key] : 0;
    out->meta[BN + tid] = key < p.tk ? p.kpos[b * p.km_bs + key] : 0;
  }
  __syncthreads();
  const uint16_t *ksu = (const uint16_t *)&ks[0][0];
  for (int u = tid; u < D * RT; u += 256) {
    const int d = u / RT, c = u % RT;
    u32x4 o = zero;
    if (c < BN / 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = ksu[vt_key(c * 8 + 2 * j) * (D + 8) + d];
        const uint32_t hi = ksu[vt_key(c * 8 + 2 * j + 1) * (D + 8) + d];
        o[j] = lo | (hi << 16);
      }
    }
    *(u32x4 *)(out->kt + u * 8) = o;
  }
}

template <int D, int DV>
__global__ __launch_bounds__(256) void bwd_pack_q_kernel(BwdParams p) {
  constexpr int QC = D / 8, GC = DV / 8;            // 16-byte data chunks per row of Q, dO
  constexpr int RN = bwd_qrow(D) / 8, RNG = bwd_qrow(DV) / 8;
  static_assert(sizeof(QTile<D, DV>) == bwd_q_tile_bytes(D, DV), "packed Q/dO tile size");
  // heads fastest: neighbouring blocks read neighbouring pieces of the same
  // token rows and of the same lines of the per-row values
  const int h = blockIdx.x, qt = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t tile = ((int64_t)b * p.hq + h) * p.tnq + qt;
  QTile<D, DV> *out = (QTile<D, DV> *)((char *)p.qpack + tile * sizeof(QTile<D, DV>));
  const bf16 *qb = (const bf16 *)p.q + b * p.q_bs + (int64_t)h * D;
  const bf16 *gb = (const bf16 *)p.dout + b * p.do_bs + (int64_t)h * DV;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // every load of this thread is issued before its first store
  constexpr int NQ = (BQ * RN + 255) / 256, NG = (BQ * RNG + 255) / 256;
  u32x4 qv[NQ], gv[NG];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int u = tid + 256 * i;
    const int r = u / RN, c = u % RN;
    const int t = qt * BQ + r;
    const bool in = u < BQ * RN && t < p.tq && c < QC;
    qv[i] = in ? *(const u32x4 *)(qb + t * p.q_ts + c * 8) : zero;
  }
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int u = tid + 256 * i;
    const int r = u / RNG, c = u % RNG;
    const int t = qt * BQ + r;
    const bool in = u < BQ * RNG && t < p.tq && c < GC;
    gv[i] = in ? *(const u32x4 *)(gb + t * p.o_ts + c * 8) : zero;
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i)
    if (tid + 256 * i < BQ * RN) *(u32x4 *)(out->qn + (tid + 256 * i) * 8) = qv[i];
#pragma unroll
  for (int i = 0; i < NG; ++i)
    if (tid + 256 * i < BQ * RNG) *(u32x4 *)(out->don + (tid + 256 * i) * 8) = gv[i];
  if (tid < BQ) {   // per-query values in the pass's query order
    const int t = qt * BQ + bwd_qperm(tid);
    const bool in = t < p.tq;
    const int64_t r = ((int64_t)b * p.tq + t) * p.hq + h;
    out->lse2[tid] = in ? p.lse2[r] : INFINITY;
    out->dsum[tid] = in ? p.dsum[r] : 0.0f;
    out->qid[tid] = in ? p.qid[b * p.qm_bs + t] : 0;
    out->qpos[tid] = in ? p.qpos[b * p.qm_bs + t] : 0;
  }
}

// ----------------------------------------------------------------------------- masks

// Visibility of one key against the lane's query (dQ pass): kid == qkey and
// lo <= qpos - kpos <= hi; a padding query gets the empty range lo > hi, so
// it sees no key whatever the ids.
struct LaneMask {
  int qkey, qpos, lo, hi;
  __device__ __forceinline__ bool operator()(int kid, int kpos) const {
    const int d = qpos - kpos;
    return (kid == qkey) & (d >= lo) & (d <= hi);
  }
};

// Visibility of one query against the lane's key (dK/dV pass): qid == kkey
// and lo <= qpos - kpos <= hi; a padding or missing key gets the empty range
// lo > hi, so no query sees it whatever the ids.
struct KeyMask {
  int kkey, kpos, lo, hi;
  __device__ __forceinline__ bool operator()(int qid, int qpos) const {
    const int d = qpos - kpos;
    return (qid == kkey) & (d >= lo) & (d <= hi);
  }
};

__device__ __forceinline__ void mask_bounds(const MaskParams &m, int &lo, int &hi) {
  lo = m.causal ? 0 : INT_MIN;
  if (m.wr >= 0) lo = max(lo, -m.wr);
  hi = m.wl >= 0 ? m.wl : INT_MAX;
}

// ----------------------------------------------------------------------------- dQ pass

template <int D, int DV, int NT, bool OUT_BF16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_dq_kernel(BwdParams p) {
  constexpr int NH = kWaves / NT;
  constexpr int BM = 32 * NT;
  constexpr int DC = D / 16;               // MFMA steps of S^T (over Q/K's head dim)
  constexpr int DCV = DV / 16;             // MFMA steps of dP^T (over V/dO's head dim)
  constexpr int DB = D / 32;
  typedef KvTile<D, DV> Tile;
  constexpr int TILE = (int)sizeof(Tile);
  constexpr int BLK = (int)offsetof(Tile, meta);   // bytes of the three bf16 blocks
  static_assert(BLK % 1024 == 0, "tile blocks are loaded 1 KB per wave instruction");
  constexpr int CHUNKS = BLK / 1024;
  constexpr int kStageBytes = kWaves * 32 * 68 * 4;
  constexpr int kSmemBytes = 2 * TILE > kStageBytes ? 2 * TILE : kStageBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  Tile &t0 = *reinterpret_cast<Tile *>(smem);
  float(*stage)[32][68] = reinterpret_cast<float(*)[32][68]>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar tile offsets
  const int col = lane & 31, half = lane >> 5;
  // Work item (xcd_item): (b, g, query tile, head chunk), head chunk fastest.
  const uint32_t hcn = (uint32_t)(p.group / NH);
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.nqt * hcn;
  const int64_t item_or_none = xcd_item(nwork, [&](uint32_t it) {
    const uint32_t r = it / hcn;   // (b, g, qt) with qt fastest
    return p.count[(r / ((uint32_t)p.nqt * (uint32_t)p.hkv)) * (uint32_t)p.nqt + r % (uint32_t)p.nqt];
  });
  if (item_or_none < 0) return;
  uint32_t w = (uint32_t)item_or_none;
  const int hc = (int)(w % hcn);
  w /= hcn;
  const int qt = (int)(w % (uint32_t)p.nqt);
  w /= (uint32_t)p.nqt;
  const int g = (int)(w % (uint32_t)p.hkv);
  const int b = (int)(w / (uint32_t)p.hkv);
  const int h = g * p.group + hc * NH + (wave % NH);
  const int tq = qt * BM + (wave / NH) * 32 + col;
  const bool qvalid = tq < p.tq;

  const int64_t row = (int64_t)b * p.nqt + qt;
  typedef const __attribute__((address_space(4))) uint32_t *const_list_t;
  const const_list_t lst = (const_list_t)(p.list + row * p.nkt);
  // read together with the count (with no key tile the list is empty and the
  // count's word stands in)
  const uint32_t e0 = *(p.nkt > 0 ? lst : (const_list_t)(p.count + row));
  // clamped so that a schedule that does not fit can never send a read past its list
  const int n = min((int)p.count[row], p.nkt);
  asm volatile("" ::"s"(e0), "s"(n));   // both loads issued before either is waited for
  const char *pack = (const char *)p.kvpack + ((int64_t)b * p.hkv + g) * p.nkt * TILE;

  auto issue = [&](Tile &dst, int kt) __attribute__((always_inline)) {
    const char *src = pack + (int64_t)kt * TILE;
#pragma unroll
    for (int i = 0; i < (CHUNKS + kWaves - 1) / kWaves; ++i) {
      const int c = wave + i * kWaves;
      if (CHUNKS % kWaves == 0 || c < CHUNKS)
        __builtin_amdgcn_global_load_lds((const void *)(src + c * 1024 + lane * 16),
                                         LDS_PTR((char *)&dst + c * 1024), 16, 0, 0);
    }
    if (wave < 2) {
      const int off = BLK + wave * (BN * 4);
      __builtin_amdgcn_global_load_lds((const void *)(src + off + lane * 4),
                                       LDS_PTR((char *)&dst + off), 4, 0, 0);
    }
  };

  // B operands: Q (for S^T = K Q^T) and dO (for dP^T = V dO^T), 8 head_dim
  // values per step.
  bf16x8 qf[DC], gf[DCV];
  {
    const bf16 *qrow = (const bf16 *)p.q + b * p.q_bs + (int64_t)tq * p.q_ts + (int64_t)h * D + 8 * half;
    const bf16 *grow = (const bf16 *)p.dout + b * p.do_bs + (int64_t)tq * p.o_ts + (int64_t)h * DV +
                       8 * half;
    const bool ld = qvalid && n > 0;
#pragma unroll
    for (int c = 0; c < DC; ++c)
      qf[c] = ld ? *(const bf16x8 *)(qrow + 16 * c) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int c = 0; c < DCV; ++c)
      gf[c] = ld ? *(const bf16x8 *)(grow + 16 * c) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  const int64_t rowidx = ((int64_t)b * p.tq + tq) * p.hq + h;
  const float l2 = qvalid ? p.lse2[rowidx] : INFINITY;
  const float dl = qvalid ? p.dsum[rowidx] : 0.0f;
  LaneMask lm;
  {
    const int my_qid = qvalid ? p.qid[b * p.qm_bs + tq] : 0;
    lm.qkey = my_qid;
    lm.qpos = qvalid ? p.qpos[b * p.qm_bs + tq] : 0;
    mask_bounds(p.mask, lm.lo, lm.hi);
    if (my_qid == 0) {   // padding (or out-of-range) query: empty window
      lm.lo = 1;
      lm.hi = 0;
    }
  }
  const bool ragged = (p.tk % BN) != 0;
  auto entry_masked = [&](uint32_t e) {
    return (e >> 31) != 0 || (ragged && (int)(e & 0x7fffffffu) == p.nkt - 1);
  };
  const float c2 = p.scale_log2;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // One 32-key block of S^T (or dP^T): A operand rows kb*32 + col of an
  // [key][d] block of NC 16-element steps, B operand the lane's query row.
  auto scores = [&](f32x16 &s, const bf16 *blk, const auto &bop) __attribute__((always_inline)) {
    constexpr int NC = sizeof(bop) / sizeof(bop[0]);
    const bf16 *arow = blk + col * (16 * NC + 8) + 8 * half;   // rows of kRowN elements
    const f32x16 zero16 = {};
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)arow, bop[0], zero16, 0, 0, 0);
#pragma unroll
    for (int c = 1; c < NC; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(arow + 16 * c), bop[c], s, 0,
                                                  0, 0);
  };

  // One tile, one 32-key block at a time: S^T and dP^T, the mask (boundary
  // tiles only), dS^T = P^T (dP^T - D) with P^T = 2^(s c2 - LSE log2 e) packed
  // to bf16 B operands, then dQ^T += K^T dS^T over the block's two 16-key chunks.
  // The next tile (next >= 0) streams into dst from between the two blocks,
  // rather than from the top of the tile, when every wave issues at once.
  auto compute = [&](const Tile &tl, bool masked, Tile &dst, int next) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
      scores(s, tl.k + kb * 32 * kRowN<D>, qf);
      scores(dp, tl.v + kb * 32 * kRowN<DV>, gf);
      if (masked) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int kk = kb * 32 + 8 * r4 + 4 * half;
          const i32x4 ids = *(const i32x4 *)&tl.meta[kk];
          const i32x4 pss = *(const i32x4 *)&tl.meta[BN + kk];
          s[4 * r4 + 0] = lm(ids.x, pss.x) ? s[4 * r4 + 0] : -INFINITY;
          s[4 * r4 + 1] = lm(ids.y, pss.y) ? s[4 * r4 + 1] : -INFINITY;
          s[4 * r4 + 2] = lm(ids.z, pss.z) ? s[4 * r4 + 2] : -INFINITY;
          s[4 * r4 + 3] = lm(ids.w, pss.w) ? s[4 * r4 + 3] : -INFINITY;
        }
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l2));
        dsf[r >> 3][r & 7] = (bf16)(pv * (dp[r] - dl));
      }
#pragma unroll
      for (int c2i = 0; c2i < 2; ++c2i) {
        const int ch = 2 * kb + c2i;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = *(const bf16x8 *)(tl.kt + (db * 32 + col) * kRowTK + 16 * ch + 8 * half);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[c2i], acc[db], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kb == 0 && next >= 0) issue(dst, next);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Double-buffered loop with one body: tile it computes from buffer it & 1
  // while tile it + 1 streams into the other (last read before the previous
  // barrier).  The list entry of tile it + 2 is loaded during tile it as a
  // vector load (the index is forced into a vector register), so the
  // end-of-tile wait covers it and no scalar load sits among the LDS reads.
  auto buffer = [&](int i) -> Tile & { return *reinterpret_cast<Tile *>(smem + i * TILE); };
  if (n > 0) {
    issue(t0, (int)(e0 & 0x7fffffffu));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  const uint32_t *lst_v = p.list + row * p.nkt;
  uint32_t ecur = e0;            // entry of tile it
  uint32_t e1v = 0;              // entry of tile it + 1, in every lane
  if (n > 1) e1v = lst_v[1];
  for (int it = 0; it < n; ++it) {
    const int cur = it & 1;
    const uint32_t e1 = __builtin_amdgcn_readfirstlane(e1v);
    const int next = it + 1 < n ? (int)(e1 & 0x7fffffffu) : -1;
    const bool masked = entry_masked(ecur);
    ecur = e1;
    if (it + 2 < n) {
      int qv = it + 2;
      asm volatile("" : "+v"(qv));
      e1v = lst_v[qv];
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(buffer(cur), masked, buffer(cur ^ 1), next);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // dQ = scale * (dQ^T)^T, through LDS in 64-column halves: 16-byte stores.
  const int tq0 = qt * BM + (wave / NH) * 32;
  const int rsub = lane >> 4, c4 = (lane & 15) * 4;
#pragma unroll
  for (int hd = 0; hd < DB / 2; ++hd) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = acc[2 * hd + j][4 * r4 + e] * p.scale;
        *(f32x4 *)&stage[wave][col][32 * j + 8 * r4 + 4 * half] = val;
      }
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int qrow = 4 * pass + rsub;
      const int t = tq0 + qrow;
      const f32x4 val = *(const f32x4 *)&stage[wave][qrow][c4];
      if (t < p.tq) {
        const int64_t rel = (int64_t)t * p.q_ts + (int64_t)h * D + 64 * hd + c4;
        if (OUT_BF16) {
          bf16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = (bf16)val[e];
          *(bf16x4 *)((bf16 *)p.dq + b * p.dq_bs + rel) = hv;
        } else {
          *(f32x4 *)((float *)p.dq + b * p.dq_bs + rel) = val;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- dK/dV pass

template <int D, int DV, bool OUT_BF16>
__global__ __launch_bounds__(64 * bwd_kv_waves(D))
__attribute__((amdgpu_waves_per_eu(bwd_kv_waves(D) / 4, bwd_kv_waves(D) / 4))) void
bwd_dkdv_kernel(BwdParams p) {
  constexpr int W = bwd_kv_waves(D);
  constexpr int KT = bwd_kv_tile(D);       // keys per workgroup
  constexpr int DC = D / 16, DCV = DV / 16;
  constexpr int DB = D / 32, DBV = DV / 32;
  typedef QTile<D, DV> Tile;
  constexpr int TILE = (int)sizeof(Tile);
  constexpr int BLK = (int)offsetof(Tile, lse2);    // bytes of the four bf16 blocks
  static_assert(BLK % 1024 == 0, "tile blocks are loaded 1 KB per wave instruction");
  constexpr int CHUNKS = BLK / 1024;
  constexpr int SROW = 68;        // staging row: 64 fp32 columns of one key, padded
  constexpr int kStageBytes = W * 32 * SROW * 4;
  constexpr int kTileBytes = 2 * TILE > kStageBytes ? 2 * TILE : kStageBytes;
  constexpr int kVBytes = W * 32 * kRowN<DV> * 2;   // the workgroup's V rows, [key][d] padded
  __shared__ __attribute__((aligned(16))) char smem[kTileBytes + kVBytes];
  Tile &t0 = *reinterpret_cast<Tile *>(smem);
  float(*stage)[32][SROW] = reinterpret_cast<float(*)[32][SROW]>(smem);
  bf16 *vrows = reinterpret_cast<bf16 *>(smem + kTileBytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar tile offsets
  const int col = lane & 31, half = lane >> 5;
  constexpr int RQ = bwd_qrow(D), RG = bwd_qrow(DV);   // Q and dO row strides in the tile
  // transpose-load position of this lane: row 4 j + half and columns
  // 16 (lane / 16 % 2) + 4 s .. + 3, where lane % 16 = 4 j + s (bwd_qperm)
  const int tr_row = 4 * ((lane & 15) >> 2) + half;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // Work item (xcd_item): (b, g, key tile), key tile fastest.
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.tnk;
  const int64_t item_or_none = xcd_item(nwork, [&](uint32_t it) {
    return p.tcount[(it / ((uint32_t)p.tnk * (uint32_t)p.hkv)) * (uint32_t)p.tnk + it % (uint32_t)p.tnk];
  });
  if (item_or_none < 0) return;
  const uint32_t item = (uint32_t)item_or_none;
  const uint32_t rest = item / (uint32_t)p.tnk;
  const int kt = (int)(item - rest * (uint32_t)p.tnk);
  const int g = (int)(rest % (uint32_t)p.hkv);
  const int b = (int)(rest / (uint32_t)p.hkv);
  const int key = kt * KT + wave * 32 + col;
  const bool kvalid = key < p.tk;

  const int64_t row = (int64_t)b * p.tnk + kt;
  typedef const __attribute__((address_space(4))) uint32_t *const_list_t;
  const const_list_t lst = (const_list_t)(p.tlist + row * p.tnq);
  // read together with the count (with no query tile the list is empty and
  // the count's word stands in)
  const uint32_t e0 = *(p.tnq > 0 ? lst : (const_list_t)(p.tcount + row));
  const int nq = min((int)p.tcount[row], p.tnq);   // clamped like the dQ pass's count
  asm volatile("" ::"s"(e0), "s"(nq));   // both loads issued before either is waited for
  const int n = nq * p.group;         // visits: (query tile, head of the group)

  // Visit it = (head it / nq of the group, query tile it % nq of the list):
  // head by head, so workgroups of neighbouring key tiles (dealt to the same
  // XCD) read the same Q tiles within a few visits of each other.
  auto entry_tile = [&](int hi, uint32_t e) {
    return ((int64_t)b * p.hq + g * p.group + hi) * p.tnq + (int)(e & 0x7fffffffu);
  };
  const bool ragged_q = (p.tq % BQ) != 0;
  auto entry_masked = [&](uint32_t e) {
    return (e >> 31) != 0 || (ragged_q && (int)(e & 0x7fffffffu) == p.tnq - 1) || !kvalid;
  };
  auto issue = [&](Tile &dst, int64_t tile) __attribute__((always_inline)) {
    const char *src = (const char *)p.qpack + tile * TILE;
#pragma unroll
    for (int i = 0; i < (CHUNKS + W - 1) / W; ++i) {
      const int c = wave + i * W;
      if (CHUNKS % W == 0 || c < CHUNKS)
        __builtin_amdgcn_global_load_lds((const void *)(src + c * 1024 + lane * 16),
                                         LDS_PTR((char *)&dst + c * 1024), 16, 0, 0);
    }
    if (wave < 2) {
      const int off = BLK + wave * 256;
      __builtin_amdgcn_global_load_lds((const void *)(src + off + lane * 4),
                                       LDS_PTR((char *)&dst + off), 4, 0, 0);
    }
  };

  // B operands: the lane's key row of K in registers, 8 head_dim values per
  // step; the wave's V rows go to LDS (row wave*32 + col, same 8-value pieces)
  // and are read back per visit, which keeps the persistent register state at
  // K plus the two accumulators.
  bf16x8 kf[DC];
  bf16 *const vmine = vrows + (wave * 32 + col) * kRowN<DV> + 8 * half;
  {
    const bf16 *krow = (const bf16 *)p.k + b * p.kv_bs + (int64_t)key * p.kv_ts + (int64_t)g * D +
                       8 * half;
    const bf16 *vrow = (const bf16 *)p.v + b * p.v_bs + (int64_t)key * p.v_ts + (int64_t)g * DV +
                       8 * half;
    const bool ld = kvalid && n > 0;
#pragma unroll
    for (int c = 0; c < DC; ++c)
      kf[c] = ld ? *(const bf16x8 *)(krow + 16 * c) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int c = 0; c < DCV; ++c)
      *(bf16x8 *)(vmine + 16 * c) =
          ld ? *(const bf16x8 *)(vrow + 16 * c) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  KeyMask km;
  {
    const int my_kid = kvalid ? p.kid[b * p.km_bs + key] : 0;
    km.kkey = my_kid;
    km.kpos = kvalid ? p.kpos[b * p.km_bs + key] : 0;
    mask_bounds(p.mask, km.lo, km.hi);
    if (my_kid == 0) {   // padding (or out-of-range) key: empty window
      km.lo = 1;
      km.hi = 0;
    }
  }
  const float c2 = p.scale_log2;

  f32x16 dk[DB], dv[DBV];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = 0.0f;
#pragma unroll
  for (int db = 0; db < DBV; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[db][r] = 0.0f;

  // dst / next: the buffer and tile of the next visit (next < 0: none), whose
  // loads are issued between P / dS and the two accumulations, so the load
  // path is busy while this wave runs its products rather than at the top of
  // the visit, when every wave issues at once.
  auto compute = [&](const Tile &tl, bool masked, Tile &dst, int64_t next) __attribute__((always_inline)) {
    // S = Q K^T and dP = dO V^T for the 32 queries of the tile: lane = key,
    // element r of the accumulator = row 8(r/4) + 4 half + r%4, which holds
    // query bwd_qperm(row) of the tile; the per-query values sit in row order.
    f32x16 s = {}, dp = {};
    {
      const int qrow = bwd_qperm(col);
      const bf16 *qa = tl.qn + qrow * RQ + 8 * half;
      const bf16 *ga = tl.don + qrow * RG + 8 * half;
      if constexpr (D == DV) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(qa + 16 * c), kf[c], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(ga + 16 * c),
                                                       *(const bf16x8 *)(vmine + 16 * c), dp, 0, 0, 0);
        }
        // operand reads three at a time, one group ahead of its two products
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int c = 0; c < DC - 1; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      } else {
#pragma unroll
        for (int c = 0; c < DC; ++c)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(qa + 16 * c), kf[c], s, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < DCV; ++c)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(ga + 16 * c),
                                                       *(const bf16x8 *)(vmine + 16 * c), dp, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (masked) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qq = 8 * r4 + 4 * half;
        const i32x4 ids = *(const i32x4 *)&tl.qid[qq];
        const i32x4 pss = *(const i32x4 *)&tl.qpos[qq];
        s[4 * r4 + 0] = km(ids.x, pss.x) ? s[4 * r4 + 0] : -INFINITY;
        s[4 * r4 + 1] = km(ids.y, pss.y) ? s[4 * r4 + 1] : -INFINITY;
        s[4 * r4 + 2] = km(ids.z, pss.z) ? s[4 * r4 + 2] : -INFINITY;
        s[4 * r4 + 3] = km(ids.w, pss.w) ? s[4 * r4 + 3] : -INFINITY;
      }
    }
    // P = 2^(s c2 - LSE log2 e), dS = P (dP - D), per query row; packed to
    // bf16 as the B operands of the two accumulations.
    bf16x8 pf[2], df[2];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int qq = 8 * r4 + 4 * half;
      const f32x4 l4 = *(const f32x4 *)&tl.lse2[qq];
      const f32x4 d4 = *(const f32x4 *)&tl.dsum[qq];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * r4 + e;
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l4[e]));
        pf[r >> 3][r & 7] = (bf16)pv;
        df[r >> 3][r & 7] = (bf16)(pv * (dp[r] - d4[e]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (next >= 0) issue(dst, next);
    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO^T P and dK^T += Q^T dS (scale applied at the end).  The A
    // operands (rows = head_dim, k = the 16 queries of step ch) are read across
    // the Q and dO rows with the transpose load: a lane of half h takes the
    // accumulator rows 16 ch + 8 r + 4 h + j (r = 0, 1; j = 0..3), the order in
    // which its P and dS values sit in the accumulator layout above, i.e. the
    // packed rows 16 ch + 4 j + 2 r + h.
    const bf16 *gtr = tl.don + tr_row * RG + tr_col;
    const bf16 *qtr = tl.qn + tr_row * RQ + tr_col;
    if constexpr (D == DV) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 ag = tr_operand(gtr + 16 * ch * RG + 32 * db, RG);
          const bf16x8 aq = tr_operand(qtr + 16 * ch * RQ + 32 * db, RQ);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, pf[ch], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, df[ch], dk[db], 0, 0, 0);
        }
      // operand loads four at a time, one group ahead of their two products
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * DB - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    } else {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
        for (int db = 0; db < DBV; ++db)
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(gtr + 16 * ch * RG + 32 * db, RG),
                                                           pf[ch], dv[db], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(qtr + 16 * ch * RQ + 32 * db, RQ),
                                                           df[ch], dk[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Double-buffered loop with one body: visit it computes from buffer it & 1
  // while visit it + 1 streams into the other (a single copy of the body keeps
  // the accumulators in one set of registers); the other buffer was last read
  // before the previous barrier.
  auto buffer = [&](int i) -> Tile & { return *reinterpret_cast<Tile *>(smem + i * TILE); };
  //
  // The list entry of visit it + 2 is loaded during visit it, as a vector load
  // (the index is forced into a vector register), so the end-of-visit wait
  // for the tile covers it and no scalar load is left in flight among the LDS
  // reads; (head, list position) advance by counters.
  if (n > 0) {
    issue(t0, entry_tile(0, e0));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  const uint32_t *lst_v = p.tlist + row * p.tnq;
  uint32_t ecur = e0;                      // entry of visit it
  int h1 = nq == 1 ? 1 : 0, q1 = nq == 1 ? 0 : 1;   // visit it + 1
  uint32_t e1v = 0;                        // its entry, in every lane
  if (n > 1) e1v = lst_v[q1];
  for (int it = 0; it < n; ++it) {
    const int cur = it & 1;
    const uint32_t e1 = __builtin_amdgcn_readfirstlane(e1v);
    const int64_t next = it + 1 < n ? entry_tile(h1, e1) : -1;
    const bool masked = entry_masked(ecur);
    ecur = e1;
    if (++q1 == nq) {
      q1 = 0;
      ++h1;
    }
    if (it + 2 < n) {
      int qv = q1;
      asm volatile("" : "+v"(qv));
      e1v = lst_v[qv];
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(buffer(cur), masked, buffer(cur ^ 1), next);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // dK = scale * (dK^T)^T and dV = (dV^T)^T through LDS: each wave stages its
  // 32 keys x 64 columns at a time, then writes 4 whole 256-byte row pieces
  // per pass, 16 bytes per lane.
  const int key0 = kt * KT + wave * 32;
  const int rsub = lane >> 4, c4 = (lane & 15) * 4;
  auto store = [&](const auto &acc, float mul, void *dst, int64_t bs, int64_t ts, int width)
      __attribute__((always_inline)) {
    constexpr int NB = sizeof(acc) / sizeof(acc[0]);   // 32-column blocks
#pragma unroll
    for (int hd = 0; hd < NB / 2; ++hd) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = acc[2 * hd + j][4 * r4 + e] * mul;
          *(f32x4 *)&stage[wave][col][32 * j + 8 * r4 + 4 * half] = val;
        }
#pragma unroll
      for (int pass = 0; pass < 8; ++pass) {
        const int kr = 4 * pass + rsub;
        const int t = key0 + kr;
        const f32x4 val = *(const f32x4 *)&stage[wave][kr][c4];
        if (t < p.tk) {
          const int64_t rel = b * bs + (int64_t)t * ts + (int64_t)g * width + 64 * hd + c4;
          if (OUT_BF16) {
            bf16x4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = (bf16)val[e];
            *(bf16x4 *)((bf16 *)dst + rel) = hv;
          } else {
            *(f32x4 *)((float *)dst + rel) = val;
          }
        }
      }
    }
  };
  __syncthreads();  // the staging reuses the tile buffers
  store(dk, p.scale, p.dk, p.dkv_bs, p.kv_ts, D);
  store(dv, 1.0f, p.dv, p.v_bs, p.v_ts, DV);
}

// ----------------------------------------------------------------------------- launchers

template <int D, int DV, int NT>
hipError_t launch_dq_nt(const BwdParams &p, bool out_bf16, hipStream_t stream) {
  constexpr int NH = kWaves / NT;
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.nqt * (p.group / NH);
  if (nwork == 0) return hipSuccess;
  const int64_t grid = (nwork + 7) / 8 * 8;
  if (out_bf16)
    hipLaunchKernelGGL((bwd_dq_kernel<D, DV, NT, true>), dim3((unsigned)grid), dim3(64 * kWaves),
                       0, stream, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, DV, NT, false>), dim3((unsigned)grid), dim3(64 * kWaves),
                       0, stream, p);
  return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_dq_d(const BwdParams &p, int32_t nt, bool out_bf16, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_dq_nt<D, DV, 1>(p, out_bf16, stream);
    case 2: return launch_dq_nt<D, DV, 2>(p, out_bf16, stream);
    case 4: return launch_dq_nt<D, DV, 4>(p, out_bf16, stream);
    case 8: return launch_dq_nt<D, DV, 8>(p, out_bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int DV>
hipError_t launch_dkdv_d(const BwdParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.tnk;
  if (nwork == 0) return hipSuccess;
  const int64_t grid = (nwork + 7) / 8 * 8;
  const dim3 block(64 * bwd_kv_waves(D));
  if (out_bf16)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DV, true>), dim3((unsigned)grid), block, 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DV, false>), dim3((unsigned)grid), block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

BwdLayout bwd_workspace_layout(int32_t batch, int32_t tq, int32_t hq, int32_t hkv, int32_t d,
                               int32_t dv, int32_t nqt, int32_t nkt, int32_t tnq, int32_t tnk) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdLayout w;
  size_t off = 0;
  const size_t B = (size_t)batch;
  w.qsum = off;   off = up(off + B * nqt * sizeof(TileSum));
  w.ksum = off;   off = up(off + B * nkt * sizeof(TileSum));
  w.count = off;  off = up(off + B * nqt * sizeof(int32_t));
  w.pairs = off;  off = up(off + B * nqt * sizeof(int64_t));
  w.list = off;   off = up(off + B * nqt * nkt * sizeof(uint32_t));
  w.tqsum = off;  off = up(off + B * tnk * sizeof(TileSum));
  w.tksum = off;  off = up(off + B * tnq * sizeof(TileSum));
  w.tcount = off; off = up(off + B * tnk * sizeof(int32_t));
  w.tpairs = off; off = up(off + B * tnk * sizeof(int64_t));
  w.tlist = off;  off = up(off + B * tnk * tnq * sizeof(uint32_t));
  w.lse2 = off;   off = up(off + B * tq * hq * sizeof(float));
  w.dsum = off;   off = up(off + B * tq * hq * sizeof(float));
  w.kvpack = off; off = up(off + B * hkv * nkt * bwd_kv_tile_bytes(d, dv));
  w.qpack = off;  off = up(off + B * hq * tnq * bwd_q_tile_bytes(d, dv));
  w.total = off;
  return w;
}

hipError_t launch_bwd_prep(const BwdParams &p, int32_t v_head_dim, bool o_bf16,
                           hipStream_t stream) {
  const int64_t tokens = (int64_t)p.batch * p.tq;
  if (tokens == 0 || p.hq == 0) return hipSuccess;
  const int64_t blocks = tokens < 65536 ? tokens : 65536;   // a token per block and pass
  const dim3 grid((unsigned)blocks);
  if (v_head_dim == 128) {
    if (o_bf16) hipLaunchKernelGGL((bwd_prep_kernel<128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_prep_kernel<128, false>), grid, dim3(256), 0, stream, p);
  } else if (v_head_dim == 64) {
    if (o_bf16) hipLaunchKernelGGL((bwd_prep_kernel<64, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_prep_kernel<64, false>), grid, dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int DV>
hipError_t pack_dd(const BwdParams &p, hipStream_t stream) {
  if (p.nkt > 0) {
    hipLaunchKernelGGL((bwd_pack_kv_kernel<D, DV>), dim3(p.nkt, p.hkv, p.batch), dim3(256), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.tnq > 0)
    hipLaunchKernelGGL((bwd_pack_q_kernel<D, DV>), dim3(p.hq, p.tnq, p.batch), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_pack(const BwdParams &p, int32_t head_dim, int32_t v_head_dim,
                           hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (head_dim == 128 && v_head_dim == 128) return pack_dd<128, 128>(p, stream);
  if (head_dim == 64 && v_head_dim == 64) return pack_dd<64, 64>(p, stream);
  if (head_dim == 192 && v_head_dim == 128) return pack_dd<192, 128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdParams &p, int32_t head_dim, int32_t v_head_dim, int32_t nt,
                         bool out_bf16, hipStream_t stream) {
  if (head_dim == 128 && v_head_dim == 128) return launch_dq_d<128, 128>(p, nt, out_bf16, stream);
  if (head_dim == 64 && v_head_dim == 64) return launch_dq_d<64, 64>(p, nt, out_bf16, stream);
  if (head_dim == 192 && v_head_dim == 128) return launch_dq_d<192, 128>(p, nt, out_bf16, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(const BwdParams &p, int32_t head_dim, int32_t v_head_dim,
                           bool out_bf16, hipStream_t stream) {
  if (head_dim == 128 && v_head_dim == 128) return launch_dkdv_d<128, 128>(p, out_bf16, stream);
  if (head_dim == 64 && v_head_dim == 64) return launch_dkdv_d<64, 64>(p, out_bf16, stream);
  if (head_dim == 192 && v_head_dim == 128) return launch_dkdv_d<192, 128>(p, out_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra
