// Tile classification and per-query-tile work lists.
//
// "Context parallelism and ring attention", section "Causal attention": a block
// of pairs that is entirely in the future (or, here, outside the window, across
// segments or in padding) is skipped, a block that is entirely valid runs
// without a mask, and only blocks that straddle a boundary are masked.
//
// Pass 1 summarises every query and key tile (counts, min/max of segment id and
// position over its valid tokens).  Pass 2, one workgroup per (batch row,
// query tile), decides each key tile from the two summaries when the ranges
// settle it and otherwise counts the tile's visible pairs exactly, so the
// classes are exact, then writes the ordered list of non-skipped key tiles
// with a partial bit, the tile classes and the query tile's visible pairs.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "internal.h"

namespace ra {

namespace {

constexpr int kMaybe = 3;

__device__ inline int wave_min(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ inline int wave_max(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ inline int wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per tile, four tiles per 256-thread block.
__global__ __launch_bounds__(256) void tile_summary_kernel(const int32_t *__restrict__ ids,
                                                           const int32_t *__restrict__ pos,
                                                           int64_t meta_bs, int32_t len,
                                                           int32_t tile, int32_t ntiles,
                                                           TileSum *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t_idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (t_idx >= ntiles) return;
  const int32_t *id_row = ids + (int64_t)b * meta_bs;
  const int32_t *pos_row = pos + (int64_t)b * meta_bs;
  int nvalid = 0, ninr = 0;
  int idmin = INT_MAX, idmax = INT_MIN, pmin = INT_MAX, pmax = INT_MIN;
  for (int i = lane; i < tile; i += 64) {
    const int t = t_idx * tile + i;
    if (t < len) {
      ++ninr;
      const int id = id_row[t];
      if (id != 0) {
        const int p = pos_row[t];
        ++nvalid;
        idmin = min(idmin, id);
        idmax = max(idmax, id);
        pmin = min(pmin, p);
        pmax = max(pmax, p);
      }
    }
  }
  nvalid = wave_sum(nvalid);
  ninr = wave_sum(ninr);
  idmin = wave_min(idmin);
  idmax = wave_max(idmax);
  pmin = wave_min(pmin);
  pmax = wave_max(pmax);
  if (lane == 0) {
    TileSum s;
    s.nvalid = nvalid;
    s.ninr = ninr;
    s.idmin = idmin;
    s.idmax = idmax;
    s.posmin = pmin;
    s.posmax = pmax;
    s.pad0 = 0;
    s.pad1 = 0;
    out[(int64_t)b * ntiles + t_idx] = s;
  }
}

// Class of a tile from the two summaries: SKIP / FULL when the ranges prove
// it, kMaybe otherwise.  Position differences are taken in 64 bits.
__device__ inline int summary_class(const TileSum &q, const TileSum &k, MaskParams m) {
  if (q.nvalid == 0 || k.nvalid == 0) return RA_TILE_SKIP;
  if (q.idmax < k.idmin || k.idmax < q.idmin) return RA_TILE_SKIP;
  const int64_t qlo = q.posmin, qhi = q.posmax, klo = k.posmin, khi = k.posmax;
  if (m.causal && klo > qhi) return RA_TILE_SKIP;
  if (m.wl >= 0 && qlo - khi > m.wl) return RA_TILE_SKIP;
  if (m.wr >= 0 && klo - qhi > m.wr) return RA_TILE_SKIP;
  const bool dense = q.nvalid == q.ninr && k.nvalid == k.ninr;
  const bool one_id = q.idmin == q.idmax && k.idmin == k.idmax && q.idmin == k.idmin;
  if (dense && one_id && (!m.causal || khi <= qlo) && (m.wl < 0 || qhi - klo <= m.wl) &&
      (m.wr < 0 || khi - qlo <= m.wr))
    return RA_TILE_FULL;
  return kMaybe;
}

__device__ inline bool visible(int qid, int qpos, int kid, int kpos, MaskParams m) {
  if (qid == 0 || qid != kid) return false;
  const int64_t d = (int64_t)qpos - (int64_t)kpos;  // query minus key position
  if (m.causal && d < 0) return false;
  if (m.wl >= 0 && d > m.wl) return false;
  if (m.wr >= 0 && -d > m.wr) return false;
  return true;
}

// grid (nqt, B), 256 threads; dynamic LDS: nkt bytes of classes.
__global__ __launch_bounds__(256) void classify_kernel(
    Schedule s, const int32_t *__restrict__ qid_all, const int32_t *__restrict__ qpos_all,
    const int32_t *__restrict__ kid_all, const int32_t *__restrict__ kpos_all, int64_t qm_bs,
    int64_t km_bs, int32_t tq, int32_t tk, int32_t bm, int32_t bn, int32_t nqt, int32_t nkt,
    MaskParams mask, int8_t *__restrict__ classes) {
  extern __shared__ uint8_t cls[];
  __shared__ int q_id_s[256], q_pos_s[256];
  __shared__ int maybe_list[256];
  __shared__ int n_maybe;
  __shared__ int tile_hits;
  __shared__ unsigned long long pair_total;
  __shared__ int scan[256];

  const int tid = threadIdx.x;
  const int qt = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t row = (int64_t)b * nqt + qt;
  const TileSum qs = s.qsum[row];
  const TileSum *ks_row = s.ksum + (int64_t)b * nkt;
  const int32_t *kid = kid_all + (int64_t)b * km_bs;
  const int32_t *kpos = kpos_all + (int64_t)b * km_bs;

  for (int i = tid; i < bm; i += 256) {
    const int t = qt * bm + i;
    q_id_s[i] = (t < tq) ? qid_all[(int64_t)b * qm_bs + t] : 0;
    q_pos_s[i] = (t < tq) ? qpos_all[(int64_t)b * qm_bs + t] : 0;
  }
  if (tid == 0) {
    n_maybe = 0;
    pair_total = 0ull;
  }
  const int chunk = (nkt + 255) / 256;
  const int k0 = min(nkt, tid * chunk), k1 = min(nkt, k0 + chunk);
  unsigned long long my_pairs = 0;
  for (int kt = k0; kt < k1; ++kt) {
    const TileSum ks = ks_row[kt];
    const int c = summary_class(qs, ks, mask);
    cls[kt] = (uint8_t)c;
    if (c == RA_TILE_FULL) my_pairs += (unsigned long long)qs.ninr * (unsigned long long)ks.ninr;
  }
  __syncthreads();
  if (my_pairs) atomicAdd(&pair_total, my_pairs);

  // Resolve undecided tiles by counting their visible pairs.
  const int pairs_per_tile = bm * bn;
  for (int base = 0; base < nkt; base += 256) {
    const int kt = base + tid;
    if (kt < nkt && cls[kt] == kMaybe) maybe_list[atomicAdd(&n_maybe, 1)] = kt;
    __syncthreads();
    const int nm = n_maybe;
    for (int j = 0; j < nm; ++j) {
      const int kt2 = maybe_list[j];
      if (tid == 0) tile_hits = 0;
      __syncthreads();
      int hits = 0;
      const int kbase = kt2 * bn;
      for (int pidx = tid; pidx < pairs_per_tile; pidx += 256) {
        const int i = pidx / bn, jj = pidx - i * bn;
        const int tq_i = qt * bm + i, tk_j = kbase + jj;
        if (tq_i < tq && tk_j < tk && visible(q_id_s[i], q_pos_s[i], kid[tk_j], kpos[tk_j], mask))
          ++hits;
      }
      hits = wave_sum(hits);
      if ((tid & 63) == 0 && hits) atomicAdd(&tile_hits, hits);
      __syncthreads();
      if (tid == 0) {
        const int h = tile_hits;
        const int inr = qs.ninr * ks_row[kt2].ninr;
        cls[kt2] = (uint8_t)(h == 0 ? RA_TILE_SKIP : (h == inr ? RA_TILE_FULL : RA_TILE_PARTIAL));
        pair_total += (unsigned long long)h;
      }
      __syncthreads();
    }
    if (tid == 0) n_maybe = 0;
    __syncthreads();
  }

  // Ordered compaction of the non-skipped key tiles.
  int mine = 0;
  for (int kt = k0; kt < k1; ++kt) mine += cls[kt] != RA_TILE_SKIP;
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  int pos = scan[tid] - mine;
  uint32_t *lst = s.list + row * (int64_t)nkt;
  for (int kt = k0; kt < k1; ++kt) {
    const int c = cls[kt];
    if (c != RA_TILE_SKIP) lst[pos++] = (uint32_t)kt | (c == RA_TILE_PARTIAL ? 0x80000000u : 0u);
  }
  if (classes) {
    int8_t *crow = classes + row * (int64_t)nkt;
    for (int kt = tid; kt < nkt; kt += 256) crow[kt] = (int8_t)cls[kt];
  }
  if (tid == 255) s.count[row] = scan[255];
  if (tid == 0) s.pairs[row] = (int64_t)pair_total;
}

__global__ __launch_bounds__(256) void pair_sum_kernel(const int64_t *__restrict__ pairs,
                                                       int32_t nqt, int64_t *__restrict__ out) {
  __shared__ unsigned long long acc;
  if (threadIdx.x == 0) acc = 0ull;
  __syncthreads();
  unsigned long long v = 0;
  const int64_t *row = pairs + (int64_t)blockIdx.x * nqt;
  for (int i = threadIdx.x; i < nqt; i += 256) v += (unsigned long long)row[i];
  atomicAdd(&acc, v);
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (int64_t)acc;
}

}  // namespace

WorkspaceLayout workspace_layout(int32_t batch, int32_t nqt, int32_t nkt, int32_t hkv,
                                 int32_t packed_head_dim, int32_t packed_v_dim) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout w;
  size_t off = 0;
  w.qsum = off;
  off = up(off + (size_t)batch * nqt * sizeof(TileSum));
  w.ksum = off;
  off = up(off + (size_t)batch * nkt * sizeof(TileSum));
  w.count = off;
  off = up(off + (size_t)batch * nqt * sizeof(int32_t));
  w.pairs = off;
  off = up(off + (size_t)batch * nqt * sizeof(int64_t));
  w.list = off;
  off = up(off + (size_t)batch * nqt * nkt * sizeof(uint32_t));
  const size_t tiles = packed_head_dim > 0 ? (size_t)batch * hkv * nkt : 0;
  const int32_t vdim = packed_v_dim > 0 ? packed_v_dim : packed_head_dim;
  w.kpack = off;
  off = up(off + tiles * (packed_head_dim > 0 ? packed_k_block_bytes(packed_head_dim) : 0));
  w.vpack = off;
  off = up(off + tiles * kBnBf16 * vdim * 2);
  w.mpack = off;
  off = up(off + tiles * 2 * kBnBf16 * sizeof(int32_t));
  w.total = off;
  return w;
}

hipError_t launch_summaries(const int32_t *ids, const int32_t *pos, int64_t meta_bs, int32_t batch,
                            int32_t len, int32_t tile, int32_t ntiles, TileSum *out,
                            hipStream_t stream) {
  if (batch == 0 || ntiles == 0) return hipSuccess;
  dim3 grid((ntiles + 3) / 4, batch);
  hipLaunchKernelGGL(tile_summary_kernel, grid, dim3(256), 0, stream, ids, pos, meta_bs, len, tile,
                     ntiles, out);
  return hipGetLastError();
}

hipError_t launch_classify(const Schedule &s, const int32_t *qid, const int32_t *qpos,
                           const int32_t *kid, const int32_t *kpos, int64_t qm_bs, int64_t km_bs,
                           int32_t batch, int32_t tq, int32_t tk, int32_t bm, int32_t bn,
                           int32_t nqt, int32_t nkt, MaskParams mask, int8_t *classes,
                           hipStream_t stream) {
  if (batch == 0 || nqt == 0) return hipSuccess;
  dim3 grid(nqt, batch);
  hipLaunchKernelGGL(classify_kernel, grid, dim3(256), (size_t)nkt, stream, s, qid, qpos, kid,
                     kpos, qm_bs, km_bs, tq, tk, bm, bn, nqt, nkt, mask, classes);
  return hipGetLastError();
}

hipError_t launch_pair_sums(const int64_t *pairs, int32_t batch, int32_t nqt, int64_t *out,
                            hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(pair_sum_kernel, dim3(batch), dim3(256), 0, stream, pairs, nqt, out);
  return hipGetLastError();
}

}  // namespace ra
