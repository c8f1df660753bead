// Work-item order shared by the forward and backward kernels (device side
// only): which item a workgroup takes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Work item of this workgroup.  Blocks are dealt to the 8 XCDs round-robin;
// each XCD takes one contiguous run of items (neighbours share K/V tiles in
// its L2), and within the run the items go longest first, so the run does not
// end on its longest items: a run whose last item has more tiles than its
// first (counts rising along the run, e.g. later queries seeing more of a
// causal window) is dealt in reverse.  Every workgroup of a run reads the same
// two counts (count_of(item) gives an item's tile count), so they agree on the
// order.  Returns -1 for a block past the last item.  One workgroup per item,
// fewer than 2^31 of them: 32-bit index arithmetic.
template <class CountOf>
__device__ __forceinline__ int64_t xcd_item(int64_t nwork, CountOf count_of) {
  const uint32_t per_xcd = gridDim.x / 8;
  const uint32_t first = (blockIdx.x % 8) * per_xcd, pos = blockIdx.x / 8;
  if ((int64_t)first >= nwork) return -1;
  const uint32_t last = (uint32_t)min((int64_t)first + per_xcd - 1, nwork - 1);
  const bool rising = count_of(last) > count_of(first);
  const uint32_t item = first + (rising ? per_xcd - 1 - pos : pos);
  return (int64_t)item < nwork ? (int64_t)item : -1;
}

}  // namespace ra
