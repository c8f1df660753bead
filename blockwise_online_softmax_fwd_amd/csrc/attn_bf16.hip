// Attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// Computes O = softmax(scale * Q K^T + M) V and the log-sum-exp of the visible
// scaled scores ("Context parallelism and ring attention", "The attention
// problem"), blockwise over 64-key tiles with the running max / sum / weighted
// sum update of its "Online softmax" section, visiting only the key tiles that
// the classification pass left in the query tile's work list ("Causal
// attention": skipped tiles never load, full tiles run unmasked).
//
// Two kernels:
//  * pack_kv: rewrites every 64-key tile of K and V (per batch row and K/V
//    head) into a contiguous, LDS-ready block: K as [key][head_dim] and V
//    transposed as [head_dim][key], 16-byte chunks XOR-swizzled by row (swz) so
//    the MFMA operand reads below are bank-conflict free, plus the tile's segment
//    ids and positions; keys past the end are zero.
//  * forward: workgroup = 8 waves = NH heads of one GQA group x NT sub-tiles
//    of 32 query tokens (NH * NT = 8).  The packed K, V^T and metadata blocks of
//    the next tile stream straight from HBM into the other half of a
//    double-buffered LDS (global_load_lds, no staging registers) while the
//    current tile computes; all NH heads read the same LDS tile.  Each wave
//    owns 32 query tokens of one head and computes transposed scores
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane then holds one query
//    column and 16 keys per 32-key block, so the row max and row sum need one
//    cross-half exchange and nothing else, and P^T is already the B operand of
//    O^T += V^T P^T (the V^T key order inside each 16-key chunk is permuted to
//    match the accumulator's row order).
//
// The running max is only raised when a new tile's max exceeds it by more than
// 2^8 in probability terms; until then probabilities up to 256 are accumulated
// against the stale max.  O = U / z and LSE = m + ln z do not depend on which
// reference max is used, and rescales of the accumulator become rare.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "bf16_tiles.h"
#include "internal.h"
#include "xcd_order.h"
#include "lse_merge.h"

namespace ra {
namespace {

using namespace tiles;

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BN = kBnBf16;          // keys per tile
constexpr float kNoMax = -1e30f;     // finite "nothing seen yet" running max
constexpr float kRescaleLog2 = 8.0f; // raise the max only beyond 2^8

// ----------------------------------------------------------------------------- packing

// Packed K rows: 64- and 128-wide rows are XOR-swizzled in place (16-byte
// chunk c of row r stored at chunk swz(r, c)); 192-wide rows (the query/key
// head dim of MLA) are padded to 200 elements instead, which spreads the 16
// rows an operand read touches over distinct banks with plain offsets.
template <int D>
struct KRow {
  static constexpr int chunks = D == 192 ? 25 : D / 8;   // 16-byte chunks per stored row
  // logical chunk held at stored chunk ph of row r (>= D/8: padding)
  __device__ static int logical(int r, int ph) {
    if constexpr (D == 192) return ph;
    else return swz<D / 8>(r, ph);
  }
  // element offset of logical chunk c within the stored row r
  __device__ static int offset(int r, int c) {
    if constexpr (D == 192) return 8 * c;
    else return 8 * swz<D / 8>(r, c);
  }
};

template <int D, int DVH>
__global__ __launch_bounds__(256) void pack_kv_kernel(PackParams p) {
  constexpr int KR = KRow<D>::chunks;      // 16-byte chunks per packed K row
  constexpr int DQC = D / 8;               // chunks of K data per row
  constexpr int VC = DVH / 8;              // chunks of V data per row
  __shared__ __attribute__((aligned(16))) bf16 vs[BN][DVH + 8];
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t tile = ((int64_t)b * p.hkv + g) * p.nkt + kt;
  const bf16 *kb = (const bf16 *)p.k + b * p.kv_bs + (int64_t)g * D;
  const bf16 *vb = (const bf16 *)p.v + b * p.v_bs + (int64_t)g * DVH;
  bf16 *kout = (bf16 *)p.kpack + tile * (BN * KR * 8);
  bf16 *vout = (bf16 *)p.vpack + tile * (BN * DVH);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  for (int u = tid; u < BN * KR; u += 256) {
    const int r = u / KR, ph = u % KR;
    const int key = kt * BN + r;
    const int lc = KRow<D>::logical(r, ph);
    u32x4 val = zero;
    if (key < p.tk && lc < DQC) val = *(const u32x4 *)(kb + key * p.kv_ts + lc * 8);
    *(u32x4 *)(kout + (int64_t)u * 8) = val;
  }
  for (int u = tid; u < BN * VC; u += 256) {
    const int r = u / VC, ph = u % VC;
    const int key = kt * BN + r;
    u32x4 vv = zero;
    if (key < p.tk) vv = *(const u32x4 *)(vb + key * p.v_ts + ph * 8);
    *(u32x4 *)&vs[r][ph * 8] = vv;
  }
  if (tid < BN) {
    const int key = kt * BN + tid;
    int32_t *meta = p.mpack + tile * (2 * BN);
    meta[tid] = key < p.tk ? p.kid[b * p.km_bs + key] : 0;
    meta[BN + tid] = key < p.tk ? p.kpos[b * p.km_bs + key] : 0;
  }
  __syncthreads();
  // V^T: DVH rows of BN keys, 8 chunks of 8 keys per row, swizzled by row.
  const uint16_t *vsu = (const uint16_t *)&vs[0][0];
  for (int u = tid; u < DVH * (BN / 8); u += 256) {
    const int d = u / (BN / 8), ph = u % (BN / 8);
    const int lc = swz<BN / 8>(d, ph);
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = vsu[vt_key(lc * 8 + 2 * j) * (DVH + 8) + d];
      const uint32_t hi = vsu[vt_key(lc * 8 + 2 * j + 1) * (DVH + 8) + d];
      out[j] = lo | (hi << 16);
    }
    *(u32x4 *)(vout + (int64_t)u * 8) = out;
  }
}

// ----------------------------------------------------------------------------- forward

// Largest of x over lanes l and l ^ 32 (the two halves of a query's keys),
// exchanged with v_permlane32_swap rather than through LDS.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// Sum of x over lanes l and l ^ 32.
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
}

// Branch-free visibility test of one key against the lane's query on a
// boundary tile: kid == qkey and lo <= qpos - kpos <= hi (lo and hi depend on
// the mask only, so they stay in scalar registers; positions are
// non-negative, so qpos - kpos cannot overflow).  qkey is the query's own
// segment id, of either sign; a padding key (id 0) never matches a live
// query.  A padding query (id 0) would match padding keys here, so its row is
// declared empty in the epilogue whatever it accumulated (a tile holding a
// padding query is never classified full).
struct LaneMask {
  int qkey, qpos, lo, hi;
  __device__ __forceinline__ bool operator()(int kid, int kpos) const {
    const int d = qpos - kpos;
    return (kid == qkey) & (d >= lo) & (d <= hi);
  }
};

template <int D, int DVH>
struct Tile {
  bf16 k[BN * KRow<D>::chunks * 8];
  bf16 vt[DVH * BN];
  int32_t meta[2 * BN];
};

// D: head dim of Q and K; DVH: head dim of V and O.
template <int D, int DVH, int NT, bool OUT_BF16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_bf16_kernel(AttnParams p) {
  constexpr int NH = kWaves / NT;
  constexpr int BM = 32 * NT;
  constexpr int DC = D / 16;               // MFMA steps over head_dim for S^T
  constexpr int DB = DVH / 32;             // 32-row blocks of O^T
  constexpr int KROW = KRow<D>::chunks * 8;
  constexpr int BLKK = BN * KROW * 2;      // bytes of one packed K block
  constexpr int BLKV = BN * DVH * 2;       // bytes of one packed V^T block
  static_assert(BLKK % 1024 == 0 && BLKV % 1024 == 0, "1 KB direct loads");
  constexpr int CK = BLKK / 1024, CV = BLKV / 1024;

  __shared__ __attribute__((aligned(16))) Tile<D, DVH> t0;
  __shared__ __attribute__((aligned(16))) Tile<D, DVH> t1;
  // Epilogue staging: each wave's 32 x 64 slice of O (fp32, rows padded to
  // 68 floats so the column-wise writes spread over the banks) and the per-row
  // weight of the running partial.
  __shared__ __attribute__((aligned(16))) float stage[kWaves][32][68];
  __shared__ float stage_w[kWaves][32];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // Work item (xcd_item): (b, g, query tile, head chunk), head chunk fastest.
  const uint32_t hcn = (uint32_t)(p.group / NH);
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.nqt * hcn;
  const int64_t item_or_none = xcd_item(nwork, [&](uint32_t it) {
    const uint32_t r = it / hcn;   // (b, g, qt) with qt fastest
    return p.count[(r / ((uint32_t)p.nqt * (uint32_t)p.hkv)) * (uint32_t)p.nqt + r % (uint32_t)p.nqt];
  });
  if (item_or_none < 0) return;
  const uint32_t item = (uint32_t)item_or_none;
  uint32_t w = item;
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
  // The work list was written by an earlier kernel and is read-only here:
  // read it through the constant address space so the loads are scalar and
  // never wait behind the direct-to-LDS tile loads.  Its first entry is read
  // together with the count (its address does not depend on the count), so
  // the first tile's load waits for one scalar round trip, not two.
  typedef const __attribute__((address_space(4))) uint32_t *const_list_t;
  const const_list_t lst = (const_list_t)(p.list + row * p.nkt);
  // (with no key tile the list is empty and the count's word stands in).  The
  // empty asm takes both values at this point, so the compiler cannot sink the
  // entry's load behind the test of the count.
  const uint32_t e0 = *(p.nkt > 0 ? lst : (const_list_t)(p.count + row));
  const int cnt = p.count[row];
  asm volatile("" ::"s"(e0), "s"(cnt));
  // clamped so that a stale schedule can only give wrong results, never an
  // access outside the packed tiles
  const int n = min(cnt, p.nkt);
  // Accumulating in place into a partial: a query tile with nothing visible in
  // this call keeps its partial as it is.
  if (p.acc_in_place && n == 0) return;
  const int64_t tile0 = ((int64_t)b * p.hkv + g) * p.nkt;
  const char *kpack = (const char *)p.kpack;
  const char *vpack = (const char *)p.vpack;
  const char *mpack = (const char *)p.mpack;

  // Direct HBM -> LDS loads of one packed tile (1 KB per wave instruction).
  auto issue = [&](Tile<D, DVH> &dst, int kt) {
    const int64_t t = tile0 + kt;
    const char *ks = kpack + t * BLKK;
    const char *vs = vpack + t * BLKV;
    if constexpr (CK % kWaves == 0 && CK == CV) {
#pragma unroll
      for (int i = 0; i < CK / kWaves; ++i) {
        const int c = wave * (CK / kWaves) + i;
        __builtin_amdgcn_global_load_lds((const void *)(ks + c * 1024 + lane * 16),
                                         LDS_PTR((char *)dst.k + c * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(vs + c * 1024 + lane * 16),
                                         LDS_PTR((char *)dst.vt + c * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < (CK + kWaves - 1) / kWaves; ++i) {
        const int c = wave + i * kWaves;
        if (c < CK)
          __builtin_amdgcn_global_load_lds((const void *)(ks + c * 1024 + lane * 16),
                                           LDS_PTR((char *)dst.k + c * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < (CV + kWaves - 1) / kWaves; ++i) {
        const int c = wave + i * kWaves;
        if (c < CV)
          __builtin_amdgcn_global_load_lds((const void *)(vs + c * 1024 + lane * 16),
                                           LDS_PTR((char *)dst.vt + c * 1024), 16, 0, 0);
      }
    }
    if (wave < 2) {
      const char *ms = mpack + t * (2 * BN * 4) + wave * (BN * 4);
      __builtin_amdgcn_global_load_lds((const void *)(ms + lane * 4),
                                       LDS_PTR((char *)dst.meta + wave * (BN * 4)), 4, 0, 0);
    }
  };

  // Q fragment (B operand of S^T = K Q^T): 8 consecutive head_dim values per step.
  bf16x8 qf[DC];
  {
    const bf16 *qrow = (const bf16 *)p.q + b * p.q_bs + (int64_t)tq * p.q_ts + (int64_t)h * D +
                       8 * half;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if (qvalid && n > 0) {
        qf[c] = *(const bf16x8 *)(qrow + 16 * c);
      } else {
        qf[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }
  // LSE of the running partial for this lane's row, read now so the epilogue
  // does not wait for it
  const float la = p.acc_mode && qvalid ? p.acc_lse[b * p.acc_lse_bs + (int64_t)tq * p.hq + h]
                                        : -INFINITY;
  LaneMask lm;
  {
    const int my_qid = qvalid ? p.qid[b * p.qm_bs + tq] : 0;
    lm.qkey = my_qid;
    lm.qpos = qvalid ? p.qpos[b * p.qm_bs + tq] : 0;
    lm.lo = p.mask.causal ? 0 : INT_MIN;
    if (p.mask.wr >= 0) lm.lo = max(lm.lo, -p.mask.wr);
    lm.hi = p.mask.wl >= 0 ? p.mask.wl : INT_MAX;
  }
  const bool ragged = (p.tk % BN) != 0;
  auto entry_tile = [&](int it) { return min((int)(lst[it] & 0x7fffffffu), p.nkt - 1); };
  auto entry_masked = [&](int it) {
    const uint32_t e = lst[it];
    return (e >> 31) != 0 || (ragged && (int)(e & 0x7fffffffu) == p.nkt - 1);
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = kNoMax;  // running max of raw scores q.k
  float z = 0.0f;    // this lane's share of the running sum
  const float c2 = p.scale_log2;

  // One tile: S^T = K Q^T, mask (boundary tiles only), online softmax, O^T += V^T P^T.
  auto compute = [&](const Tile<D, DVH> &tl, bool masked) {
    f32x16 s[2];
    {
      bf16x8 ka0[DC], ka1[DC];
      const bf16 *krow0 = tl.k + col * KROW, *krow1 = tl.k + (32 + col) * KROW;
#pragma unroll
      for (int c = 0; c < DC; ++c) ka0[c] = *(const bf16x8 *)(krow0 + KRow<D>::offset(col, 2 * c + half));
#pragma unroll
      for (int c = 0; c < DC; ++c) ka1[c] = *(const bf16x8 *)(krow1 + KRow<D>::offset(col, 2 * c + half));
      const f32x16 zero16 = {};
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0[0], qf[0], zero16, 0, 0, 0);
#pragma unroll
      for (int c = 1; c < DC; ++c)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0[c], qf[c], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1[0], qf[0], zero16, 0, 0, 0);
#pragma unroll
      for (int c = 1; c < DC; ++c)
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1[c], qf[c], s[1], 0, 0, 0);
      // all of block 0's operand reads first, then block 1's reads one per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, DC, 0);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, DC, 0);
    }
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int kk = kb * 32 + 8 * r4 + 4 * half;
          const i32x4 ids = *(const i32x4 *)&tl.meta[kk];
          const i32x4 pss = *(const i32x4 *)&tl.meta[BN + kk];
          s[kb][4 * r4 + 0] = lm(ids.x, pss.x) ? s[kb][4 * r4 + 0] : -INFINITY;
          s[kb][4 * r4 + 1] = lm(ids.y, pss.y) ? s[kb][4 * r4 + 1] : -INFINITY;
          s[kb][4 * r4 + 2] = lm(ids.z, pss.z) ? s[kb][4 * r4 + 2] : -INFINITY;
          s[kb][4 * r4 + 3] = lm(ids.w, pss.w) ? s[kb][4 * r4 + 3] : -INFINITY;
        }
    }

    // V^T operands of this tile: issued now, consumed after the exps.
    bf16x8 va[DB][4];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16 *vrow = tl.vt + (db * 32 + col) * BN;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) va[db][ch] = *(const bf16x8 *)(vrow + 8 * swz<BN / 8>(col, 2 * ch + half));
    }
    // Row max over this tile (the lane's 32 keys, then the other half's).
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    const bool raise = (mx - m) * c2 > kRescaleLog2;
    if (__ballot(raise)) {
      if (raise) {
        const float alpha = __builtin_amdgcn_exp2f((m - mx) * c2);
        m = mx;
        z *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    const float mc = m * c2;

    // P^T = exp2(s * c2 - m * c2), summed and packed to bf16 B operands.
    bf16x8 pf[4];
    float zs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -mc));
        zs += pv;
        pf[kb * 2 + (r >> 3)][r & 7] = (bf16)pv;
      }
    z += zs;

    // O^T += V^T P^T, chunk by chunk so chunk ch's MFMAs can start while the
    // exps of chunk ch+1 are still running.
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][ch], pf[ch], o[db], 0, 0, 0);
  };

  // Double-buffered loop, unrolled by two so each half names its LDS buffer
  // statically: while tile it computes from one buffer, tile it+1 streams
  // into the other.
  if (n > 0) {
    issue(t0, min((int)(e0 & 0x7fffffffu), p.nkt - 1));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  for (int it = 0; it < n;) {
    if (it + 1 < n) issue(t1, entry_tile(it + 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(t0, entry_masked(it));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (++it >= n) break;
    if (it + 1 < n) issue(t0, entry_tile(it + 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(t1, entry_masked(it));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    ++it;
  }

  // Epilogue: O = U / z, LSE = scale * m + ln z; empty rows get 0 and -inf.
  // With a running partial (O_a, L_a): L = log(e^LSE + e^L_a) and
  // O = e^(LSE - L) U / z + e^(L_a - L) O_a.
  // The wave's O^T fragment goes through LDS in two 64-column halves so that
  // every global access of O and O_a is a contiguous 16-byte piece of a row.
  // O is stored with the non-temporal hint: it is not read again by this
  // launch, and streaming it keeps the L2 for the K/V tiles that neighbouring
  // workgroups share.
  const float zt = pair_sum(z);
  const bool live = zt > 0.0f && lm.qkey != 0;   // padding queries see nothing
  const float l_own = live ? p.scale * m + logf(zt) : -INFINITY;
  float w_own = live ? 1.0f / zt : 0.0f;
  float w_acc = 0.0f, l_out = l_own;
  if (p.acc_mode && qvalid) {
    l_out = lse_add(l_own, la);
    w_acc = lse_weight(la, l_out);
    w_own = live ? lse_weight(l_own, l_out) / zt : 0.0f;
  }
  if (qvalid && half == 0)
    p.lse[b * p.lse_bs + (int64_t)tq * p.hq + h + (tq >= p.o_split ? p.lse_split_off : 0)] = l_out;
  if (half == 0) stage_w[wave][col] = w_acc;

  const int tq0 = qt * BM + (wave / NH) * 32;   // first query token of this wave
  const int rsub = lane >> 4;                   // row within a group of 4 rows
  const int c4 = (lane & 15) * 4;               // first of this lane's 4 columns
  // The running partial of the pieces this lane writes, loaded before any of
  // them is stored so the loads are in flight together (in place, a lane
  // reads exactly the addresses it later writes); rows whose partial is empty
  // (weight 0) are not read.  Both halves at once where registers allow
  // (MLA's kernel has none to spare: one half at a time there).
  constexpr int PH = D == 192 ? 1 : DB / 2;   // halves loaded up front
  f32x4 acc[DB / 2][8];
  auto load_half = [&](int hd) {
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int t = tq0 + 4 * pass + rsub;
      const int64_t rel = (int64_t)t * p.o_ts + (int64_t)h * DVH + 64 * hd + c4;
      f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
      if (t < p.tq && stage_w[wave][4 * pass + rsub] != 0.0f) {
        if (p.acc_mode == 2) {
          const bf16x4 ah = *(const bf16x4 *)((const bf16 *)p.acc_o + b * p.acc_o_bs + rel);
          a[0] = (float)ah[0];
          a[1] = (float)ah[1];
          a[2] = (float)ah[2];
          a[3] = (float)ah[3];
        } else {
          a = *(const f32x4 *)((const float *)p.acc_o + b * p.acc_o_bs + rel);
        }
      }
      acc[hd][pass] = a;
    }
  };
  if (p.acc_mode) {
#pragma unroll
    for (int hd = 0; hd < PH; ++hd) load_half(hd);
  }
#pragma unroll
  for (int hd = 0; hd < DB / 2; ++hd) {
    if (hd >= PH && p.acc_mode) load_half(hd);
    // fragment columns of db = 2*hd, 2*hd+1 -> stage[wave][query][0..63]
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 val;
        val[0] = o[2 * hd + j][4 * r4 + 0] * w_own;
        val[1] = o[2 * hd + j][4 * r4 + 1] * w_own;
        val[2] = o[2 * hd + j][4 * r4 + 2] * w_own;
        val[3] = o[2 * hd + j][4 * r4 + 3] * w_own;
        *(f32x4 *)&stage[wave][col][32 * j + 8 * r4 + 4 * half] = val;
      }
    // read back 4 rows x 64 columns per pass, 16 bytes per lane
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int qrow = 4 * pass + rsub;
      const int t = tq0 + qrow;
      f32x4 val = *(const f32x4 *)&stage[wave][qrow][c4];
      if (t < p.tq) {
        const int64_t rel = (int64_t)t * p.o_ts + (int64_t)h * DVH + 64 * hd + c4;
        const int64_t orel = rel + (t >= p.o_split ? p.o_split_off : 0);   // split output
        const float wa = stage_w[wave][qrow];
        if (wa != 0.0f) val += wa * acc[hd][pass];
        if (OUT_BF16) {
          bf16x4 hv;
          hv[0] = (bf16)val[0];
          hv[1] = (bf16)val[1];
          hv[2] = (bf16)val[2];
          hv[3] = (bf16)val[3];
          __builtin_nontemporal_store(hv, (bf16x4 *)((bf16 *)p.o + b * p.o_bs + orel));
        } else {
          __builtin_nontemporal_store(val, (f32x4 *)((float *)p.o + b * p.o_bs + orel));
        }
      }
    }
  }
}

template <int D, int DVH, int NT>
hipError_t launch_nt(const AttnParams &p, bool out_bf16, hipStream_t stream) {
  constexpr int NH = kWaves / NT;
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.nqt * (p.group / NH);
  if (nwork == 0) return hipSuccess;
  const int64_t grid = (nwork + 7) / 8 * 8;
  if (out_bf16)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, DVH, NT, true>), dim3((unsigned)grid), dim3(512),
                       0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, DVH, NT, false>), dim3((unsigned)grid), dim3(512),
                       0, stream, p);
  return hipGetLastError();
}

template <int D, int DVH>
hipError_t launch_d(const AttnParams &p, int32_t nt, bool out_bf16, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_nt<D, DVH, 1>(p, out_bf16, stream);
    case 2: return launch_nt<D, DVH, 2>(p, out_bf16, stream);
    case 4: return launch_nt<D, DVH, 4>(p, out_bf16, stream);
    case 8: return launch_nt<D, DVH, 8>(p, out_bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t packed_k_block_bytes(int32_t head_dim) {
  return (size_t)BN * (head_dim == 192 ? 200 : head_dim) * 2;
}

hipError_t launch_pack_kv(const PackParams &p, int32_t head_dim, int32_t v_head_dim,
                          hipStream_t stream) {
  if (p.batch == 0 || p.nkt == 0) return hipSuccess;
  dim3 grid(p.nkt, p.hkv, p.batch);
  if (head_dim == 128 && v_head_dim == 128)
    hipLaunchKernelGGL((pack_kv_kernel<128, 128>), grid, dim3(256), 0, stream, p);
  else if (head_dim == 64 && v_head_dim == 64)
    hipLaunchKernelGGL((pack_kv_kernel<64, 64>), grid, dim3(256), 0, stream, p);
  else if (head_dim == 192 && v_head_dim == 128)
    hipLaunchKernelGGL((pack_kv_kernel<192, 128>), grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnParams &p, int32_t head_dim, int32_t v_head_dim, int32_t nt,
                            bool out_bf16, hipStream_t stream) {
  if (head_dim == 128 && v_head_dim == 128) return launch_d<128, 128>(p, nt, out_bf16, stream);
  if (head_dim == 64 && v_head_dim == 64) return launch_d<64, 64>(p, nt, out_bf16, stream);
  if (head_dim == 192 && v_head_dim == 128) return launch_d<192, 128>(p, nt, out_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra
