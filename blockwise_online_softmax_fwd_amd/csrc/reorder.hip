// Causal load-balancing permutation of the sequence axis (TransformerEngine JAX
// tutorial, section 4: reorder_causal_load_balancing and its inverse, seq_dim 1).
//
// Both directions are gathers, so every row is written exactly once with
// sequential stores:  forward dst[b, p] = src[b, map(p)],
// inverse dst[b, o] = src[b, map^-1(o)].  Rows are opaque bytes, moved in the
// widest unit (16, 8, 4, 2 or 1 bytes) that the row size and both base
// pointers allow.  Wide rows (q, k, v, o: kilobytes each) get a block per row
// segment; narrow rows (ids, positions, lse) one thread per unit.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "reorder_map.h"

namespace ra {
namespace {

template <typename U>
__global__ __launch_bounds__(256) void reorder_wide_kernel(const U *__restrict__ src,
                                                           U *__restrict__ dst, int32_t seq,
                                                           int64_t units, int32_t cp,
                                                           int32_t kind, int32_t stripe,
                                                           int32_t inverse) {
  const int64_t row = blockIdx.x;  // b * seq + p (destination row)
  const int64_t b = row / seq;
  const int64_t pdst = row - b * seq;
  const int64_t psrc = inverse ? reorder_dst(pdst, seq, cp, kind, stripe)
                               : reorder_src(pdst, seq, cp, kind, stripe);
  const U *s = src + (b * seq + psrc) * units;
  U *d = dst + row * units;
  for (int64_t u = (int64_t)blockIdx.y * 1024 + threadIdx.x; u < units;
       u += (int64_t)gridDim.y * 1024) {
    U x0 = s[u];
    U x1, x2, x3;
    const bool h1 = u + 256 < units, h2 = u + 512 < units, h3 = u + 768 < units;
    if (h1) x1 = s[u + 256];
    if (h2) x2 = s[u + 512];
    if (h3) x3 = s[u + 768];
    d[u] = x0;
    if (h1) d[u + 256] = x1;
    if (h2) d[u + 512] = x2;
    if (h3) d[u + 768] = x3;
  }
}

template <typename U>
__global__ __launch_bounds__(256) void reorder_narrow_kernel(const U *__restrict__ src,
                                                             U *__restrict__ dst, int64_t rows,
                                                             int32_t seq, int32_t units,
                                                             int32_t cp, int32_t kind,
                                                             int32_t stripe, int32_t inverse) {
  const int64_t total = rows * units;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / units;
    const int64_t u = i - row * units;
    const int64_t b = row / seq;
    const int64_t pdst = row - b * seq;
    const int64_t psrc = inverse ? reorder_dst(pdst, seq, cp, kind, stripe)
                                 : reorder_src(pdst, seq, cp, kind, stripe);
    dst[i] = src[(b * seq + psrc) * units + u];
  }
}

struct alignas(16) U16 {
  uint32_t x[4];
};
struct alignas(8) U8 {
  uint32_t x[2];
};

template <typename U>
hipError_t go(const void *src, void *dst, int32_t batch, int32_t seq, int64_t row_bytes, int32_t cp,
              int32_t kind, int32_t stripe, int32_t inverse, hipStream_t stream) {
  const int64_t units = row_bytes / (int64_t)sizeof(U);
  const int64_t rows = (int64_t)batch * seq;
  if (units >= 256) {
    int64_t gy = (units + 1023) / 1024;
    if (gy > 65535) gy = 65535;
    hipLaunchKernelGGL(reorder_wide_kernel<U>, dim3((unsigned)rows, (unsigned)gy), dim3(256), 0,
                       stream, (const U *)src, (U *)dst, seq, units, cp, kind, stripe, inverse);
  } else {
    int64_t blocks = (rows * units + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(reorder_narrow_kernel<U>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const U *)src, (U *)dst, rows, seq, (int32_t)units, cp, kind, stripe,
                       inverse);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reorder(const void *src, void *dst, int32_t batch, int32_t seq, int64_t row_bytes,
                          int32_t cp, int32_t kind, int32_t stripe, bool inverse,
                          hipStream_t stream) {
  if (batch == 0 || seq == 0) return hipSuccess;
  const uintptr_t align = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
  const int inv = inverse ? 1 : 0;
  if ((align & 15) == 0) return go<U16>(src, dst, batch, seq, row_bytes, cp, kind, stripe, inv, stream);
  if ((align & 7) == 0) return go<U8>(src, dst, batch, seq, row_bytes, cp, kind, stripe, inv, stream);
  if ((align & 3) == 0) return go<uint32_t>(src, dst, batch, seq, row_bytes, cp, kind, stripe, inv, stream);
  if ((align & 1) == 0) return go<uint16_t>(src, dst, batch, seq, row_bytes, cp, kind, stripe, inv, stream);
  return go<uint8_t>(src, dst, batch, seq, row_bytes, cp, kind, stripe, inv, stream);
}

}  // namespace ra
