// Attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// Computes O = softmax(scale * Q K^T + M) V and the log-sum-exp of the visible
// scaled scores ("Context parallelism and ring attention", "The attention
// problem"), blockwise over 64-key tiles with the running max / sum / weighted
// sum update of its "Online softmax" section, visiting only the key tiles that
// the classification pass left in the query tile's work list ("Causal
// attention": skipped tiles never load, full tiles run unmasked).
//
// Workgroup: 8 waves = NH heads of one GQA group x NT sub-tiles of 32 query
// tokens (NH * NT = 8).  All waves share one K tile and one V tile in LDS, so
// every K/V byte brought on chip feeds NH heads.  Each wave owns 32 query
// tokens of one head and works on transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16: a lane then holds one query column and 16 keys per
// 32-key block, so the row max and row sum need one cross-half exchange and no
// other lane traffic, and the transposed probabilities P^T are already laid out
// as the B operand of O^T += V^T P^T.  V is written to LDS transposed, with the
// keys of every 16-key chunk permuted to match that operand's lane layout, so
// every MFMA operand read is one 16-byte LDS load.
//
// The running max is only raised when a new tile's max exceeds it by more than
// 2^8 in probability terms; until then probabilities up to 256 are accumulated
// against the stale max.  O = U / z and LSE = m + ln z are unchanged by which
// reference max is used, and rescales of the 64-float accumulator become rare.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = kBnBf16;    // keys per tile
constexpr int KPAD = 8;        // bf16 padding per K row (row stride 4 mod 64 banks)
constexpr int VPAD = 8;        // bf16 padding per V^T row
constexpr float kNoMax = -1e30f;         // finite "nothing seen yet" running max
constexpr float kRescaleLog2 = 8.0f;     // raise the max only beyond 2^8

template <int D>
struct Smem {
  bf16 k[2][BN][D + KPAD];
  bf16 vt[2][D][BN + VPAD];
  int kid[2][BN];
  int kpos[2][BN];
};

// LDS column of key kk (0..63) inside its V^T row: within each 16-key chunk a
// lane of half h reads 8 consecutive columns 8h..8h+7, which must hold keys
// 4h..4h+3 and 8+4h..8+4h+3 (the rows that half holds in the score accumulator).
__device__ __forceinline__ int vt_col(int kk) {
  return (kk & ~15) + ((kk >> 2) & 1) * 8 + ((kk >> 3) & 1) * 4 + (kk & 3);
}

__device__ __forceinline__ bool visible(int qid, int qpos, int kid, int kpos, const MaskParams &m) {
  if (qid == 0 || qid != kid) return false;
  const int64_t d = (int64_t)qpos - (int64_t)kpos;
  if (m.causal && d < 0) return false;
  if (m.wl >= 0 && d > m.wl) return false;
  if (m.wr >= 0 && -d > m.wr) return false;
  return true;
}

template <int D, int NT, bool OUT_BF16>
__global__ __launch_bounds__(512) void attn_fwd_bf16_kernel(AttnParams p) {
  constexpr int NH = kWaves / NT;
  constexpr int BM = 32 * NT;
  constexpr int DC = D / 16;          // MFMA steps over head_dim for S^T
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int DV = D / 8;           // 16-byte chunks per K/V row
  constexpr int KU = BN * DV;         // K tile units of 16 bytes
  constexpr int KPT = (KU + 511) / 512;
  constexpr int VU = (BN / 2) * DV;   // V tile units: 2 keys x 16 bytes
  static_assert(VU <= 512, "one V unit per thread");

  __shared__ Smem<D> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // Work item, with consecutive items kept on one XCD (blocks are dealt to the
  // 8 XCDs round-robin; each XCD gets one contiguous run of items).
  const int hcn = p.group / NH;
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.nqt * hcn;
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (item >= nwork) return;
  int64_t w = item;
  const int hc = (int)(w % hcn);
  w /= hcn;
  const int qt = (int)(w % p.nqt);
  w /= p.nqt;
  const int g = (int)(w % p.hkv);
  const int b = (int)(w / p.hkv);

  const int h = g * p.group + hc * NH + (wave % NH);
  const int tq = qt * BM + (wave / NH) * 32 + col;
  const bool qvalid = tq < p.tq;

  // Q fragment (B operand of S^T = K Q^T): 8 consecutive head_dim values per step.
  bf16x8 qf[DC];
  {
    const bf16 *qrow = (const bf16 *)p.q + b * p.q_bs + (int64_t)tq * p.hq * D + (int64_t)h * D +
                       8 * half;
    for (int c = 0; c < DC; ++c) {
      if (qvalid) {
        qf[c] = *(const bf16x8 *)(qrow + 16 * c);
      } else {
        for (int e = 0; e < 8; ++e) qf[c][e] = (bf16)0.0f;
      }
    }
  }
  const int my_qid = qvalid ? p.qid[b * p.qm_bs + tq] : 0;
  const int my_qpos = qvalid ? p.qpos[b * p.qm_bs + tq] : 0;

  const int64_t row = (int64_t)b * p.nqt + qt;
  const int n = p.count[row];
  const uint32_t *lst = p.list + row * p.nkt;

  const bf16 *kbase = (const bf16 *)p.k + b * p.kv_bs + (int64_t)g * D;
  const bf16 *vbase = (const bf16 *)p.v + b * p.kv_bs + (int64_t)g * D;
  const int32_t *kid_row = p.kid + b * p.km_bs;
  const int32_t *kpos_row = p.kpos + b * p.km_bs;
  const int64_t kv_tok = (int64_t)p.hkv * D;
  const bool ragged = (p.tk % BN) != 0;

  bf16x8 kreg[KPT];
  bf16x8 vreg0, vreg1;
  int idreg = 0, posreg = 0;

  auto load_tile = [&](int kt) {
    for (int i = 0; i < KPT; ++i) {
      const int u = tid + 512 * i;
      if (u < KU) {
        const int r = u / DV, dc = u % DV;
        const int key = kt * BN + r;
        if (key < p.tk) {
          kreg[i] = *(const bf16x8 *)(kbase + key * kv_tok + dc * 8);
        } else {
          for (int e = 0; e < 8; ++e) kreg[i][e] = (bf16)0.0f;
        }
      }
    }
    if (tid < VU) {
      const int dc = tid % DV, kp = tid / DV;
      const int key0 = kt * BN + 2 * kp;
      if (key0 < p.tk) {
        vreg0 = *(const bf16x8 *)(vbase + key0 * kv_tok + dc * 8);
      } else {
        for (int e = 0; e < 8; ++e) vreg0[e] = (bf16)0.0f;
      }
      if (key0 + 1 < p.tk) {
        vreg1 = *(const bf16x8 *)(vbase + (key0 + 1) * kv_tok + dc * 8);
      } else {
        for (int e = 0; e < 8; ++e) vreg1[e] = (bf16)0.0f;
      }
    }
    if (tid < BN) {
      const int key = kt * BN + tid;
      idreg = key < p.tk ? kid_row[key] : 0;
      posreg = key < p.tk ? kpos_row[key] : 0;
    }
  };

  auto store_tile = [&](int buf) {
    for (int i = 0; i < KPT; ++i) {
      const int u = tid + 512 * i;
      if (u < KU) {
        const int r = u / DV, dc = u % DV;
        *(bf16x8 *)&sm.k[buf][r][dc * 8] = kreg[i];
      }
    }
    if (tid < VU) {
      const int dc = tid % DV, kp = tid / DV;
      const int c = vt_col(2 * kp);
      for (int e = 0; e < 8; ++e) {
        union {
          bf16 h2[2];
          uint32_t u;
        } pk;
        pk.h2[0] = vreg0[e];
        pk.h2[1] = vreg1[e];
        *(uint32_t *)&sm.vt[buf][dc * 8 + e][c] = pk.u;
      }
    }
    if (tid < BN) {
      sm.kid[buf][tid] = idreg;
      sm.kpos[buf][tid] = posreg;
    }
  };

  f32x16 o[DB];
  for (int db = 0; db < DB; ++db)
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = kNoMax;   // running max of raw scores q.k
  float z = 0.0f;     // this lane's share of the running sum
  const float c2 = p.scale_log2;

  if (n > 0) {
    load_tile((int)(lst[0] & 0x7fffffffu));
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n; ++it) {
    const uint32_t e = lst[it];
    const int kt = (int)(e & 0x7fffffffu);
    const bool masked = (e >> 31) || (ragged && kt == p.nkt - 1);
    const int buf = it & 1;
    if (it + 1 < n) load_tile((int)(lst[it + 1] & 0x7fffffffu));

    // S^T for the two 32-key blocks.
    f32x16 s[2];
    for (int kb = 0; kb < 2; ++kb) {
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      for (int c = 0; c < DC; ++c) {
        const bf16x8 a = *(const bf16x8 *)&sm.k[buf][kb * 32 + col][16 * c + 8 * half];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    }
    if (masked) {
      for (int kb = 0; kb < 2; ++kb)
        for (int r4 = 0; r4 < 4; ++r4) {
          const int kk = kb * 32 + 8 * r4 + 4 * half;
          const int4 ids = *(const int4 *)&sm.kid[buf][kk];
          const int4 pss = *(const int4 *)&sm.kpos[buf][kk];
          if (!visible(my_qid, my_qpos, ids.x, pss.x, p.mask)) s[kb][4 * r4 + 0] = -INFINITY;
          if (!visible(my_qid, my_qpos, ids.y, pss.y, p.mask)) s[kb][4 * r4 + 1] = -INFINITY;
          if (!visible(my_qid, my_qpos, ids.z, pss.z, p.mask)) s[kb][4 * r4 + 2] = -INFINITY;
          if (!visible(my_qid, my_qpos, ids.w, pss.w, p.mask)) s[kb][4 * r4 + 3] = -INFINITY;
        }
    }

    // Row max over this tile (the lane's 32 keys, then the other half's).
    float mx = s[0][0];
    for (int kb = 0; kb < 2; ++kb)
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool raise = (mx - m) * c2 > kRescaleLog2;
    if (__ballot(raise)) {
      if (raise) {
        const float alpha = __builtin_amdgcn_exp2f((m - mx) * c2);
        m = mx;
        z *= alpha;
        for (int db = 0; db < DB; ++db)
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    const float mc = m * c2;

    // P^T = exp2(s * c2 - m * c2), summed and packed to bf16 B operands.
    bf16x8 pf[4];
    float zs = 0.0f;
    for (int kb = 0; kb < 2; ++kb)
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -mc));
        zs += pv;
        pf[kb * 2 + (r >> 3)][r & 7] = (bf16)pv;
      }
    z += zs;

    // O^T += V^T P^T over the four 16-key chunks.
    for (int db = 0; db < DB; ++db)
      for (int ch = 0; ch < 4; ++ch) {
        const bf16x8 a = *(const bf16x8 *)&sm.vt[buf][db * 32 + col][ch * 16 + 8 * half];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], o[db], 0, 0, 0);
      }

    if (it + 1 < n) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = U / z, LSE = scale * m + ln z; empty rows get 0 and -inf.
  const float zt = z + __shfl_xor(z, 32);
  if (!qvalid) return;
  const bool live = zt > 0.0f;
  const float inv = live ? 1.0f / zt : 0.0f;
  const int64_t obase = b * p.o_bs + (int64_t)tq * p.hq * D + (int64_t)h * D + 4 * half;
  for (int db = 0; db < DB; ++db)
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + 8 * r4;
      f32x4 val;
      val[0] = o[db][4 * r4 + 0] * inv;
      val[1] = o[db][4 * r4 + 1] * inv;
      val[2] = o[db][4 * r4 + 2] * inv;
      val[3] = o[db][4 * r4 + 3] * inv;
      if (OUT_BF16) {
        bf16x4 hv;
        hv[0] = (bf16)val[0];
        hv[1] = (bf16)val[1];
        hv[2] = (bf16)val[2];
        hv[3] = (bf16)val[3];
        *(bf16x4 *)((bf16 *)p.o + obase + d) = hv;
      } else {
        *(f32x4 *)((float *)p.o + obase + d) = val;
      }
    }
  if (half == 0)
    p.lse[b * p.lse_bs + (int64_t)tq * p.hq + h] = live ? p.scale * m + logf(zt) : -INFINITY;
}

template <int D, int NT>
hipError_t launch_nt(const AttnParams &p, bool out_bf16, hipStream_t stream) {
  constexpr int NH = kWaves / NT;
  const int64_t nwork = (int64_t)p.batch * p.hkv * p.nqt * (p.group / NH);
  if (nwork == 0) return hipSuccess;
  const int64_t grid = (nwork + 7) / 8 * 8;
  if (out_bf16)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NT, true>), dim3((unsigned)grid), dim3(512), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NT, false>), dim3((unsigned)grid), dim3(512), 0,
                       stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams &p, int32_t nt, bool out_bf16, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_nt<D, 1>(p, out_bf16, stream);
    case 2: return launch_nt<D, 2>(p, out_bf16, stream);
    case 4: return launch_nt<D, 4>(p, out_bf16, stream);
    case 8: return launch_nt<D, 8>(p, out_bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams &p, int32_t head_dim, int32_t nt, bool out_bf16,
                            hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(p, nt, out_bf16, stream);
  if (head_dim == 64) return launch_d<64>(p, nt, out_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra
