// LDS tile layouts shared by the bf16 forward and backward kernels (device
// side only): vector types, the XOR swizzle of 16-byte chunks and the key
// order of transposed operand blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {
namespace tiles {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Per-token ids and positions are read from LDS as this vector type, not as
// HIP's int4 struct: the compiler puts a wait for every LDS DMA in flight in
// front of a struct read, but not in front of a vector read.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Token (0..15) stored at column x (0..15) of a 16-token chunk of a transposed
// block.  In the accumulator of v_mfma_f32_32x32x16_bf16 a lane of half h holds
// rows 4h..4h+3 and 8+4h..8+4h+3 of every 16-row group; packed to bf16 they
// are that lane's 8 k-values of the next product, so the A operand's columns
// 8h..8h+7 must hold exactly those tokens.
__device__ __forceinline__ int vt_key(int x) {
  const int h = (x >> 3) & 1, e = x & 7;
  return (x & ~15) + (e < 4 ? 4 * h + e : 8 + 4 * h + (e - 4));
}

// XOR swizzle of the 16-byte chunks of a packed row.  LDS serves a 16-byte
// read for 16 lanes per cycle across 256 bytes of banks; the MFMA operand
// reads have 16 lanes on 16 consecutive rows at the same logical chunk, so the
// physical chunk is XORed with the row's index among the rows that share one
// 256-byte bank line.  CPR = 16-byte chunks per row (4, 8 or 16).
template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "rows of 64, 128 or 256 bytes");
  return CPR == 16 ? (chunk ^ (row & 15))
                   : (CPR == 8 ? (chunk ^ ((row >> 1) & 7)) : (chunk ^ ((row >> 2) & 3)));
}

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

}  // namespace tiles
}  // namespace ra
