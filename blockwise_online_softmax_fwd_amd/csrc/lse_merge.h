// Log-sum-exp merge of two partial results over disjoint key sets
// ("Context parallelism and ring attention", "Online softmax", written over
// (output, log-sum-exp) pairs): L = log(e^a + e^b), and a partial with
// log-sum-exp l enters the merged output with weight e^(l - L).  A partial
// with l = -inf (no visible key) has weight 0; if both are -inf, L = -inf.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace ra {

__device__ __forceinline__ float lse_add(float a, float b) {
  if (a == -INFINITY) return b;
  if (b == -INFINITY) return a;
  return fmaxf(a, b) + log1pf(expf(-fabsf(a - b)));
}

__device__ __forceinline__ float lse_weight(float l, float total) {
  return l == -INFINITY ? 0.0f : expf(l - total);
}

}  // namespace ra
