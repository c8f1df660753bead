// Merge of two partial attention results over disjoint key sets.
//
// "Context parallelism and ring attention", section "Online softmax": a new
// block's (m_b, z_b, u_b) folds into the running (m, z, u) with weights
// exp(m - m') and exp(m_b - m').  A partial result here is (O, LSE) with
// O = u / z and LSE = m + ln z, i.e. the state (LSE, 1, O), and the fold reads
//   LSE = log(exp(LSE_a) + exp(LSE_b)),
//   O   = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b.
// Rows with no visible key (LSE = -inf) are the identity of the merge; two such
// rows give O = 0, LSE = -inf.
//
// HBM-bound: each (batch, token, head) row reads two D-vectors and two LSE
// values and writes one D-vector and one LSE.  One thread moves 4 consecutive
// elements (16 bytes of fp32 or 8 of bf16); D/4 threads share a row, and a
// thread issues the loads of four rows before it combines any of them.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ f32x4 load4(const void *base, int64_t off) {
  if (BF) {
    const bf16x4 v = *(const bf16x4 *)((const __bf16 *)base + off);
    f32x4 r;
    r[0] = (float)v[0];
    r[1] = (float)v[1];
    r[2] = (float)v[2];
    r[3] = (float)v[3];
    return r;
  }
  return *(const f32x4 *)((const float *)base + off);
}

template <bool BF>
__device__ __forceinline__ void store4(void *base, int64_t off, f32x4 v) {
  if (BF) {
    bf16x4 h;
    h[0] = (__bf16)v[0];
    h[1] = (__bf16)v[1];
    h[2] = (__bf16)v[2];
    h[3] = (__bf16)v[3];
    *(bf16x4 *)((__bf16 *)base + off) = h;
  } else {
    *(f32x4 *)((float *)base + off) = v;
  }
}

template <int D, bool ABF, bool BBF, bool OBF>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;        // threads per row
  constexpr int RPB = 256 / TPR;    // rows per block and step
  constexpr int U = 4;              // rows per thread per iteration, loads issued together
  const int64_t rows_per_batch = (int64_t)p.seq * p.heads;
  const int64_t total = rows_per_batch * p.batch;
  const int sub = threadIdx.x % TPR;
  const int64_t step = (int64_t)gridDim.x * RPB * U;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U + threadIdx.x / TPR; r0 < total; r0 += step) {
    float la[U], lb[U];
    f32x4 a[U], c[U];
    int64_t bb[U], rr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + (int64_t)u * RPB;
      bb[u] = r / rows_per_batch;
      rr[u] = r - bb[u] * rows_per_batch;
      if (r < total) {
        la[u] = p.la[bb[u] * p.la_bs + rr[u]];
        lb[u] = p.lb[bb[u] * p.lb_bs + rr[u]];
        const int64_t col = rr[u] * D + sub * 4;
        a[u] = load4<ABF>(p.oa, bb[u] * p.oa_bs + col);
        c[u] = load4<BBF>(p.ob, bb[u] * p.ob_bs + col);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + (int64_t)u * RPB;
      if (r >= total) break;
      // A side at -inf contributes nothing and its O is never read into the
      // result (select, not multiply), so an empty row is the identity.
      const bool ea = la[u] == -INFINITY, eb = lb[u] == -INFINITY;
      const float mx = fmaxf(la[u], lb[u]);
      float lo = mx + log1pf(expf(-fabsf(la[u] - lb[u])));
      const float wa = expf(la[u] - lo), wb = expf(lb[u] - lo);
      f32x4 out = wa * a[u] + wb * c[u];
      if (eb) { out = a[u]; lo = la[u]; }
      if (ea) { out = c[u]; lo = lb[u]; }
      if (ea && eb) { out = f32x4{0.0f, 0.0f, 0.0f, 0.0f}; lo = -INFINITY; }
      store4<OBF>(p.oo, bb[u] * p.oo_bs + rr[u] * D + sub * 4, out);
      if (sub == 0) p.lo[bb[u] * p.lo_bs + rr[u]] = lo;
    }
  }
}

template <int D, bool ABF, bool BBF, bool OBF>
hipError_t launch4(const MergeParams &p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.seq * p.heads;
  if (rows == 0) return hipSuccess;
  constexpr int RPB = 256 / (D / 4) * 4;  // rows per block and iteration
  int64_t blocks = (rows + RPB - 1) / RPB;
  const int64_t cap = 256 * 64;  // enough blocks to fill 256 CUs many times over
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((merge_kernel<D, ABF, BBF, OBF>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const MergeParams &p, int a, int b, int o, hipStream_t s) {
  const int key = (a == RA_BF16) * 4 + (b == RA_BF16) * 2 + (o == RA_BF16);
  switch (key) {
    case 0: return launch4<D, false, false, false>(p, s);
    case 1: return launch4<D, false, false, true>(p, s);
    case 2: return launch4<D, false, true, false>(p, s);
    case 3: return launch4<D, false, true, true>(p, s);
    case 4: return launch4<D, true, false, false>(p, s);
    case 5: return launch4<D, true, false, true>(p, s);
    case 6: return launch4<D, true, true, false>(p, s);
    default: return launch4<D, true, true, true>(p, s);
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams &p, int32_t a_dtype, int32_t b_dtype, int32_t out_dtype,
                        hipStream_t stream) {
  if (p.d == 128) return launch_d<128>(p, a_dtype, b_dtype, out_dtype, stream);
  if (p.d == 64) return launch_d<64>(p, a_dtype, b_dtype, out_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra
