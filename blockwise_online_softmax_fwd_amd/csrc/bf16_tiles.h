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

}  // namespace tiles
}  // namespace ra
