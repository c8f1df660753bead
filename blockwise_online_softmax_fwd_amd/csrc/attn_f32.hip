// Attention forward for fp32 Q/K/V (no reduced-precision step anywhere).
//
// Same computation and work lists as the bf16 path ("Context parallelism and
// ring attention": "The attention problem", "Online softmax", "Causal
// attention"), on the vector ALUs: every query token is handled by a pair of
// lanes that each hold half of head_dim of q and of the running output; the
// key tile (32 keys) and value tile live in LDS and are read as broadcasts.
// Scores, probabilities and the running max / sum stay in fp32 and the running
// max is exact (raised on every increase).
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"
#include "lse_merge.h"

namespace ra {
namespace {

constexpr int BM = kBmF32;
constexpr int BN = kBnF32;

__device__ __forceinline__ bool visible(int qid, int qpos, int kid, int kpos, const MaskParams &m) {
  if (qid == 0 || qid != kid) return false;
  const int64_t d = (int64_t)qpos - (int64_t)kpos;
  if (m.causal && d < 0) return false;
  if (m.wl >= 0 && d > m.wl) return false;
  if (m.wr >= 0 && -d > m.wr) return false;
  return true;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int DH = D / 2;
  __shared__ float ks[BN][D + 4];
  __shared__ float vs[BN][D + 4];
  __shared__ int kid_s[BN], kpos_s[BN];

  const int tid = threadIdx.x;
  const int tok = tid >> 1, half = tid & 1;
  int64_t w = blockIdx.x;
  const int qt = (int)(w % p.nqt);
  w /= p.nqt;
  const int h = (int)(w % p.hq);
  const int b = (int)(w / p.hq);
  const int g = h / p.group;
  const int tq = qt * BM + tok;
  const bool qvalid = tq < p.tq;

  float q[DH], o[DH];
  const float *qrow = (const float *)p.q + b * p.q_bs + (int64_t)tq * p.q_ts + (int64_t)h * D +
                      half * DH;
  for (int d = 0; d < DH; ++d) {
    q[d] = qvalid ? qrow[d] : 0.0f;
    o[d] = 0.0f;
  }
  const int my_qid = qvalid ? p.qid[b * p.qm_bs + tq] : 0;
  const int my_qpos = qvalid ? p.qpos[b * p.qm_bs + tq] : 0;

  const int64_t row = (int64_t)b * p.nqt + qt;
  // clamped so that a stale schedule can only give wrong results, never an
  // access outside K and V
  const int n = min(p.count[row], p.nkt);
  if (p.acc_in_place && n == 0) return;  // partial stays as it is
  const uint32_t *lst = p.list + row * p.nkt;
  const float *kb = (const float *)p.k + b * p.kv_bs + (int64_t)g * D;
  const float *vb = (const float *)p.v + b * p.v_bs + (int64_t)g * D;
  const int64_t kv_tok = p.kv_ts;
  const bool ragged = (p.tk % BN) != 0;

  float m = -INFINITY, z = 0.0f;
  for (int it = 0; it < n; ++it) {
    const uint32_t e = lst[it];
    const int kt = min((int)(e & 0x7fffffffu), p.nkt - 1);
    const bool masked = (e >> 31) || (ragged && kt == p.nkt - 1);
    __syncthreads();
    for (int u = tid; u < BN * D; u += 128) {
      const int r = u / D, d = u % D;
      const int key = kt * BN + r;
      ks[r][d] = key < p.tk ? kb[key * kv_tok + d] : 0.0f;
      vs[r][d] = key < p.tk ? vb[key * p.v_ts + d] : 0.0f;
    }
    if (tid < BN) {
      const int key = kt * BN + tid;
      kid_s[tid] = key < p.tk ? p.kid[b * p.km_bs + key] : 0;
      kpos_s[tid] = key < p.tk ? p.kpos[b * p.km_bs + key] : 0;
    }
    __syncthreads();

    float sc[BN];
    float mx = -INFINITY;
    for (int j = 0; j < BN; ++j) {
      float part = 0.0f;
      for (int d = 0; d < DH; ++d) part = fmaf(q[d], ks[j][half * DH + d], part);
      float s = (part + __shfl_xor(part, 1)) * p.scale;
      if (masked && !visible(my_qid, my_qpos, kid_s[j], kpos_s[j], p.mask)) s = -INFINITY;
      sc[j] = s;
      mx = fmaxf(mx, s);
    }
    if (mx > m) {
      const float alpha = expf(m - mx);  // m = -inf gives 0
      z *= alpha;
      for (int d = 0; d < DH; ++d) o[d] *= alpha;
      m = mx;
    }
    if (m == -INFINITY) continue;
    for (int j = 0; j < BN; ++j) {
      const float pj = expf(sc[j] - m);
      z += pj;
      for (int d = 0; d < DH; ++d) o[d] = fmaf(pj, vs[j][half * DH + d], o[d]);
    }
  }

  if (!qvalid) return;
  const bool live = z > 0.0f;
  const float l_own = live ? m + logf(z) : -INFINITY;
  float w_own = live ? 1.0f / z : 0.0f;
  float w_acc = 0.0f, l_out = l_own;
  const int64_t rel = (int64_t)tq * p.o_ts + (int64_t)h * D + half * DH;
  if (p.acc_mode) {
    const float la = p.acc_lse[b * p.acc_lse_bs + (int64_t)tq * p.hq + h];
    l_out = lse_add(l_own, la);
    w_acc = lse_weight(la, l_out);
    w_own = live ? lse_weight(l_own, l_out) / z : 0.0f;
  }
  const int64_t obase = b * p.o_bs + rel + (tq >= p.o_split ? p.o_split_off : 0);  // split output
  const int64_t abase = b * p.acc_o_bs + rel;
  for (int d = 0; d < DH; ++d) {
    float val = o[d] * w_own;
    if (w_acc != 0.0f) {
      const float a = p.acc_mode == 2 ? (float)((const __bf16 *)p.acc_o)[abase + d]
                                      : ((const float *)p.acc_o)[abase + d];
      val += w_acc * a;
    }
    if (OUT_BF16)
      ((__bf16 *)p.o)[obase + d] = (__bf16)val;
    else
      ((float *)p.o)[obase + d] = val;
  }
  if (half == 0)
    p.lse[b * p.lse_bs + (int64_t)tq * p.hq + h + (tq >= p.o_split ? p.lse_split_off : 0)] = l_out;
}

template <int D>
hipError_t launch_d(const AttnParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t nwork = (int64_t)p.batch * p.hq * p.nqt;
  if (nwork == 0) return hipSuccess;
  if (out_bf16)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, true>), dim3((unsigned)nwork), dim3(128), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, false>), dim3((unsigned)nwork), dim3(128), 0, stream,
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
