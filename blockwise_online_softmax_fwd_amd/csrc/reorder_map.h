// Causal load-balancing sequence maps, shared by the host index query and the
// device reorder kernel so both always agree.
//
// A map sends a reordered position p to the original position map(p); after
// reordering, rank r owns the contiguous shard [r*n, (r+1)*n), n = T / R.
//  * dual chunk ("Context parallelism and ring attention", "Load balance": pair
//    an early and a late piece on each device): T is cut into 2R stripes of
//    c = T / (2R) tokens; the first c slots of shard r hold stripe r, the next
//    c slots hold stripe 2R-1-r.
//  * striped (TransformerEngine JAX tutorial, section 4, ReorderStrategy.Striped
//    with stripe_size s): stripe j of s tokens belongs to rank j mod R; shard r
//    lists its stripes in increasing j.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define RA_HD __host__ __device__ inline
#else
#define RA_HD inline
#endif

namespace ra {

// original position of reordered slot p
RA_HD int64_t reorder_src(int64_t p, int64_t t, int32_t r, int32_t kind, int32_t s) {
  const int64_t n = t / r;
  const int64_t rank = p / n;
  const int64_t w = p - rank * n;
  if (kind == 0) {
    const int64_t c = t / (2 * r);
    const int64_t stripe = (w < c) ? rank : (2 * (int64_t)r - 1 - rank);
    return stripe * c + (w < c ? w : w - c);
  }
  const int64_t j = (w / s) * r + rank;
  return j * s + (w % s);
}

// reordered slot of original position o (inverse of reorder_src)
RA_HD int64_t reorder_dst(int64_t o, int64_t t, int32_t r, int32_t kind, int32_t s) {
  const int64_t n = t / r;
  if (kind == 0) {
    const int64_t c = t / (2 * r);
    const int64_t stripe = o / c;
    const int64_t within = o - stripe * c;
    if (stripe < r) return stripe * n + within;
    return (2 * (int64_t)r - 1 - stripe) * n + c + within;
  }
  const int64_t j = o / s;
  const int64_t within = o - j * s;
  const int64_t rank = j % r;
  return rank * n + (j / r) * s + within;
}

}  // namespace ra
