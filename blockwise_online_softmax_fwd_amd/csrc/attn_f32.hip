// Attention forward for fp32 Q/K/V on gfx950 matrix cores, with no
// reduced-precision step anywhere.
//
// Same computation and work lists as the bf16 path ("Context parallelism and
// ring attention": "The attention problem", "Online softmax", "Causal
// attention"), on the fp32 matrix instruction v_mfma_f32_32x32x2_f32: fp32
// operands, fp32 accumulation.  A work item is 64 query tokens of one head
// (two waves of 32) against the 32-key tiles of its work list; each tile's K
// and V rows go through LDS, where both waves read them.
//
// Per wave and tile:
//  * S^T = K Q^T (32 keys x 32 queries).  MFMA k-step c takes head_dim index c
//    from the lanes of half 0 and c + D/2 from those of half 1, so a lane's
//    operands of four consecutive steps are four consecutive floats of its
//    K row (one 16-byte LDS read) and of its Q row (registers).  A lane then
//    holds one query column and 16 of the 32 keys; the row max and sum need
//    one cross-half exchange.
//  * P^T = exp2(S^T scale log2(e) - m scale log2(e)) stays where the
//    accumulator put it: k-step j of O^T += V^T P^T takes, from the lane's
//    half h, the key 8 (j / 4) + 4 h + j % 4, which is exactly the lane's
//    P element j.
//  * O^T is D/32 blocks of 32 rows; row m of block db is head_dim index
//    (D/32) m + db, so one LDS read of D/32 consecutive floats of a V row
//    gives the A operands of all blocks, and at the end a lane's accumulator
//    element r holds D/32 consecutive outputs of its query row, stored as one
//    piece.
// The running max is raised lazily (only beyond 2^8 in probability terms), as
// in the bf16 kernel: O = U / z and LSE = m + ln z do not depend on which
// reference max is used.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "internal.h"
#include "xcd_order.h"
#include "lse_merge.h"

namespace ra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kBmF32;           // query tokens per work item (two waves)
constexpr int BN = kBnF32;           // keys per tile
constexpr float kNoMax = -1e30f;     // finite "nothing seen yet" running max
constexpr float kRescaleLog2 = 8.0f; // raise the max only beyond 2^8

// Largest / sum of x over lanes l and l ^ 32 (the two halves of a query's keys).
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
}

// Visibility of one key against the lane's query on a boundary tile:
// kid == qkey and lo <= qpos - kpos <= hi.  qkey is the query's own segment id;
// a padding query (id 0) would match padding keys here, so its row is declared
// empty in the epilogue (a tile holding a padding query is never classified
// full, so it always passes through this test).
struct LaneMask {
  int qkey, qpos, lo, hi;
  __device__ __forceinline__ bool operator()(int kid, int kpos) const {
    const int d = qpos - kpos;
    return (kid == qkey) & (d >= lo) & (d <= hi);
  }
};

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_f32_kernel(AttnParams p) {
  constexpr int DH = D / 2;   // MFMA k-steps of S^T
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  // LDS row stride: 16 lanes reading 16 bytes of 16 consecutive rows start
  // 4 * 33 (D = 128) or 4 * 17 (D = 64) words apart, which is 4 banks apart
  // modulo 64: no conflict.
  constexpr int KT = D + 4;
  __shared__ __attribute__((aligned(16))) float ks[BN * KT];
  __shared__ __attribute__((aligned(16))) float vs[BN * KT];
  __shared__ int32_t kid_s[BN], kpos_s[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  // Work item (xcd_item): (b, h, query tile), query tile fastest.
  const int64_t nwork = (int64_t)p.batch * p.hq * p.nqt;
  const int64_t item_or_none = xcd_item(nwork, [&](uint32_t it) {
    return p.count[(it / ((uint32_t)p.nqt * (uint32_t)p.hq)) * (uint32_t)p.nqt + it % (uint32_t)p.nqt];
  });
  if (item_or_none < 0) return;
  uint32_t w = (uint32_t)item_or_none;
  const int qt = (int)(w % (uint32_t)p.nqt);
  w /= (uint32_t)p.nqt;
  const int h = (int)(w % (uint32_t)p.hq);
  const int b = (int)(w / (uint32_t)p.hq);
  const int g = h / p.group;
  const int tq = qt * BM + wave * 32 + col;
  const bool qvalid = tq < p.tq;

  const int64_t row = (int64_t)b * p.nqt + qt;
  // clamped so that a stale schedule can only give wrong results, never an
  // access outside K and V
  const int n = min(p.count[row], p.nkt);
  if (p.acc_in_place && n == 0) return;  // the partial stays as it is
  const uint32_t *lst = p.list + row * p.nkt;

  // Q (B operand of S^T): element c of the lane's half is head_dim index c + half * DH
  float qf[DH];
  {
    const float *qrow = (const float *)p.q + b * p.q_bs + (int64_t)tq * p.q_ts + (int64_t)h * D +
                        half * DH;
#pragma unroll
    for (int c4 = 0; c4 < DH / 4; ++c4) {
      const f32x4 v4 = qvalid && n > 0 ? *(const f32x4 *)(qrow + 4 * c4) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      qf[4 * c4 + 0] = v4[0];
      qf[4 * c4 + 1] = v4[1];
      qf[4 * c4 + 2] = v4[2];
      qf[4 * c4 + 3] = v4[3];
    }
  }
  LaneMask lm;
  lm.qkey = qvalid ? p.qid[b * p.qm_bs + tq] : 0;
  lm.qpos = qvalid ? p.qpos[b * p.qm_bs + tq] : 0;
  lm.lo = p.mask.causal ? 0 : INT_MIN;
  if (p.mask.wr >= 0) lm.lo = max(lm.lo, -p.mask.wr);
  lm.hi = p.mask.wl >= 0 ? p.mask.wl : INT_MAX;

  const float *kb = (const float *)p.k + b * p.kv_bs + (int64_t)g * D;
  const float *vb = (const float *)p.v + b * p.v_bs + (int64_t)g * D;
  const bool ragged = (p.tk % BN) != 0;
  const float c2 = p.scale_log2;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = kNoMax;  // running max of raw scores q.k
  float z = 0.0f;    // this lane's share of the running sum

  for (int it = 0; it < n; ++it) {
    const uint32_t e = lst[it];
    const int kt = min((int)(e & 0x7fffffffu), p.nkt - 1);
    const bool masked = (e >> 31) || (ragged && kt == p.nkt - 1);
    __syncthreads();   // both waves are done with the previous tile
    // K and V rows of the tile (keys past the end are zero), 16 bytes per step
#pragma unroll 4
    for (int u = tid; u < BN * (D / 4); u += 128) {
      const int r = u / (D / 4), c4 = u % (D / 4);
      const int key = kt * BN + r;
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 kv = key < p.tk ? *(const f32x4 *)(kb + (int64_t)key * p.kv_ts + 4 * c4) : zero;
      const f32x4 vv = key < p.tk ? *(const f32x4 *)(vb + (int64_t)key * p.v_ts + 4 * c4) : zero;
      *(f32x4 *)&ks[r * KT + 4 * c4] = kv;
      *(f32x4 *)&vs[r * KT + 4 * c4] = vv;
    }
    if (tid < BN) {
      const int key = kt * BN + tid;
      kid_s[tid] = key < p.tk ? p.kid[b * p.km_bs + key] : 0;
      kpos_s[tid] = key < p.tk ? p.kpos[b * p.km_bs + key] : 0;
    }
    __syncthreads();

    // S^T = K Q^T in two accumulation chains (even / odd groups of four steps)
    f32x16 sa = {}, sb = {};
    const float *krow = ks + col * KT + half * DH;
#pragma unroll
    for (int c4 = 0; c4 < DH / 4; ++c4) {
      const f32x4 a = *(const f32x4 *)(krow + 4 * c4);
      f32x16 &acc = (c4 & 1) ? sb : sa;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], qf[4 * c4 + j], acc, 0, 0, 0);
    }
    f32x16 s = sa + sb;
    // element r of s: key 8 (r / 4) + 4 half + r % 4 of the tile
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * half + (r & 3);
        s[r] = lm(kid_s[key], kpos_s[key]) ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
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
    float pv[16];
    float zs = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pv[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
      zs += pv[r];
    }
    z += zs;

    // O^T += V^T P^T: step j takes key 8 (j / 4) + 4 half + j % 4 (the lane's
    // P element j); block db's row col is head_dim index DB * col + db.
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + 4 * half + (j & 3);
      const float *vrow = vs + key * KT + DB * col;
      if constexpr (DB == 4) {
        const f32x4 a = *(const f32x4 *)vrow;
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[db], pv[j], o[db], 0, 0, 0);
      } else {
        const f32x2 a = *(const f32x2 *)vrow;
#pragma unroll
        for (int db = 0; db < 2; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[db], pv[j], o[db], 0, 0, 0);
      }
    }
  }

  // Epilogue: O = U / z, LSE = scale * m + ln z; empty rows get 0 and -inf.
  // With a running partial (O_a, L_a): L = log(e^LSE + e^L_a) and
  // O = e^(LSE - L) U / z + e^(L_a - L) O_a.
  const float zt = pair_sum(z);
  if (!qvalid) return;
  const bool live = zt > 0.0f && lm.qkey != 0;   // padding queries see nothing
  const float l_own = live ? p.scale * m + logf(zt) : -INFINITY;
  float w_own = live ? 1.0f / zt : 0.0f;
  float w_acc = 0.0f, l_out = l_own;
  if (p.acc_mode) {
    const float la = p.acc_lse[b * p.acc_lse_bs + (int64_t)tq * p.hq + h];
    l_out = lse_add(l_own, la);
    w_acc = lse_weight(la, l_out);
    w_own = live ? lse_weight(l_own, l_out) / zt : 0.0f;
  }
  if (half == 0)
    p.lse[b * p.lse_bs + (int64_t)tq * p.hq + h + (tq >= p.o_split ? p.lse_split_off : 0)] = l_out;
  const int64_t rel = (int64_t)tq * p.o_ts + (int64_t)h * D;
  const int64_t obase = b * p.o_bs + rel + (tq >= p.o_split ? p.o_split_off : 0);   // split output
  const int64_t abase = b * p.acc_o_bs + rel;
  // element r of every block: head_dim indices DB * (8 (r / 4) + 4 half + r % 4) + db
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int d0 = DB * (8 * (r >> 2) + 4 * half + (r & 3));
    float val[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) val[db] = o[db][r] * w_own;
    if (w_acc != 0.0f) {
      if (p.acc_mode == 2) {
        const __bf16 *ap = (const __bf16 *)p.acc_o + abase + d0;
#pragma unroll
        for (int db = 0; db < DB; ++db) val[db] += w_acc * (float)ap[db];
      } else {
        const float *ap = (const float *)p.acc_o + abase + d0;
#pragma unroll
        for (int db = 0; db < DB; ++db) val[db] += w_acc * ap[db];
      }
    }
    if constexpr (OUT_BF16) {
      __bf16 *op = (__bf16 *)p.o + obase + d0;
      if constexpr (DB == 4) {
        *(bf16x4 *)op = bf16x4{(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
      } else {
        *(bf16x2 *)op = bf16x2{(__bf16)val[0], (__bf16)val[1]};
      }
    } else {
      float *op = (float *)p.o + obase + d0;
      if constexpr (DB == 4) {
        *(f32x4 *)op = f32x4{val[0], val[1], val[2], val[3]};
      } else {
        *(f32x2 *)op = f32x2{val[0], val[1]};
      }
    }
  }
}

template <int D>
hipError_t launch_d(const AttnParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t nwork = (int64_t)p.batch * p.hq * p.nqt;
  if (nwork == 0) return hipSuccess;
  const int64_t grid = (nwork + 7) / 8 * 8;   // whole runs for the 8 XCDs (xcd_item)
  if (out_bf16)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, true>), dim3((unsigned)grid), dim3(128), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, false>), dim3((unsigned)grid), dim3(128), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams &p, int32_t head_dim, bool out_bf16,
                           hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(p, out_bf16, stream);
  if (head_dim == 64) return launch_d<64>(p, out_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra
