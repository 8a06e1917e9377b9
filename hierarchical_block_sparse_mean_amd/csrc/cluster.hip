// Query clusters: the (query, slot) entries of every head are grouped by the
// key block they must score or attend ("Block Sparse Attention with
// Log-Linear Complexity", hyper.ai page, section "kernel implementation":
// queries that need the same candidate key block form a cluster, and each
// cluster is cut into tiles).
//
// Counting sort in three passes, no global atomics:
//   1. per tile of 8192 entries, an LDS histogram over the head's key blocks;
//   2. per (head, bin), a running sum down the tiles gives the bin total and
//      each tile's base within the bin; per head, an exclusive scan over the
//      bins gives each bin's first pair; then one scan of the work-chunk
//      counts of all clusters;
//   3. per tile, an LDS cursor per bin scatters the pair code (t << 5) | slot.
// Heads with more key blocks than the LDS histogram holds use a global-atomic
// fallback.  Either way: counts[c], offsets[c] (first pair) and
// chunk_off[c] (first work chunk, chunk_off[ncl] = total) for c = head*M + j.
#include "kernels.h"

namespace pisa {

constexpr int kHistTile = 8192;     // entries per histogram tile
constexpr int64_t kMaxBins = 16384; // LDS bins (64 KB)

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t cluster_scratch_bytes(int64_t heads, int64_t NK, int64_t M) {
  if (M > kMaxBins) return 256;
  const int64_t tiles = (NK + kHistTile - 1) / kHistTile;
  return al256(sizeof(int32_t) * (size_t)heads * tiles * M);
}

__global__ void hist_kernel(const int32_t* __restrict__ keys, int64_t NK, int64_t M, int64_t tiles,
                            int32_t* __restrict__ hist) {
  extern __shared__ int32_t s_h[];
  const int64_t head = blockIdx.y, tile = blockIdx.x;
  for (int64_t i = threadIdx.x; i < M; i += blockDim.x) s_h[i] = 0;
  __syncthreads();
  const int64_t lo = head * NK + tile * kHistTile;
  const int64_t hi = (tile + 1) * kHistTile < NK ? lo + kHistTile : head * NK + NK;
  for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x) {
    const int32_t j = keys[e];
    if (j >= 0 && j < M) atomicAdd(&s_h[j], 1);
  }
  __syncthreads();
  int32_t* out = hist + (head * tiles + tile) * M;
  for (int64_t i = threadIdx.x; i < M; i += blockDim.x) out[i] = s_h[i];
}

// Per (head, bin), one thread: a running sum down the tiles turns each
// histogram entry into the position of that tile's first pair relative to the
// bin's first pair, and gives the bin total.
__global__ void col_scan_kernel(int32_t* hist, int64_t M, int64_t tiles, int32_t* counts) {
  const int64_t head = blockIdx.y;
  const int64_t bin = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (bin >= M) return;
  int32_t* hh = hist + head * tiles * M + bin;
  int32_t run = 0;
  for (int64_t tl = 0; tl < tiles; tl += 8) {
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = tl + u < tiles ? hh[(tl + u) * M] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (tl + u < tiles) {
        hh[(tl + u) * M] = run;
        run += c[u];
      }
  }
  counts[head * M + bin] = run;
}

// One workgroup per head: offsets = head * NK + exclusive scan of the bin
// totals.
__global__ __launch_bounds__(1024) void bin_scan_kernel(const int32_t* __restrict__ counts, int64_t NK, int64_t M,
                                                        int32_t* offsets) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_carry;
  const int64_t head = blockIdx.x;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < M; base += 1024) {
    const int64_t bin = base + threadIdx.x;
    const int32_t v = bin < M ? counts[head * M + bin] : 0;
    s_part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? s_part[threadIdx.x - o] : 0;
      __syncthreads();
      s_part[threadIdx.x] += add;
      __syncthreads();
    }
    if (bin < M) offsets[head * M + bin] = (int32_t)(head * NK) + s_carry + s_part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry += s_part[1023];
    __syncthreads();
  }
}

// pair code of entry e_loc = t * K + slot of a head: (t << 5) | slot (K <= 32)
__device__ __forceinline__ int32_t pair_code(int64_t e_loc, int32_t K) {
  const int32_t t = (int32_t)(e_loc / K);
  return (t << 5) | (int32_t)(e_loc - (int64_t)t * K);
}

__global__ void scatter_kernel(const int32_t* __restrict__ keys, int64_t NK, int32_t K, int64_t M, int64_t tiles,
                               const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
                               int32_t* __restrict__ pairs) {
  extern __shared__ int32_t s_cur[];
  const int64_t head = blockIdx.y, tile = blockIdx.x;
  const int32_t* b = base + (head * tiles + tile) * M;
  for (int64_t i = threadIdx.x; i < M; i += blockDim.x) s_cur[i] = offsets[head * M + i] + b[i];
  __syncthreads();
  const int64_t lo = head * NK + tile * kHistTile;
  const int64_t hi = (tile + 1) * kHistTile < NK ? lo + kHistTile : head * NK + NK;
  for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x) {
    const int32_t j = keys[e];
    if (j >= 0 && j < M) pairs[atomicAdd(&s_cur[j], 1)] = pair_code(e - head * NK, K);
  }
}

// Single-workgroup exclusive scan of the work-chunk counts of all clusters.
__global__ __launch_bounds__(1024) void chunk_scan_kernel(const int32_t* __restrict__ counts, int64_t ncl,
                                                          int32_t chunk, int32_t* chunk_off) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < ncl; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int32_t v = i < ncl ? (counts[i] + chunk - 1) / chunk : 0;
    s_part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? s_part[threadIdx.x - o] : 0;
      __syncthreads();
      s_part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < ncl) chunk_off[i] = s_carry + s_part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry += s_part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) chunk_off[ncl] = s_carry;
}

// ---- fallback for heads with more than kMaxBins key blocks ----------------------
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void atomic_count_kernel(const int32_t* __restrict__ keys, int64_t entries, int64_t NK, int64_t M,
                                    int32_t* counts) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < entries;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t j = keys[e];
    if (j >= 0 && j < M) atomicAdd(&counts[(e / NK) * M + j], 1);
  }
}

// offsets[c] = exclusive scan of counts (contiguous over all clusters)
__global__ __launch_bounds__(1024) void offset_scan_kernel(const int32_t* __restrict__ counts, int64_t ncl,
                                                           int32_t* offsets) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < ncl; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int32_t v = i < ncl ? counts[i] : 0;
    s_part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? s_part[threadIdx.x - o] : 0;
      __syncthreads();
      s_part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < ncl) offsets[i] = s_carry + s_part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry += s_part[1023];
    __syncthreads();
  }
}

__global__ void atomic_fill_kernel(const int32_t* __restrict__ keys, int64_t entries, int64_t NK, int32_t K,
                                   int64_t M, const int32_t* __restrict__ offsets, int32_t* cursor,
                                   int32_t* pairs) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < entries;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t j = keys[e];
    if (j < 0 || j >= M) continue;
    const int64_t c = (e / NK) * M + j;
    pairs[offsets[c] + atomicAdd(&cursor[c], 1)] = pair_code(e % NK, K);
  }
}

hipError_t launch_clusters(const int32_t* keys, int64_t heads, int64_t NK, int32_t K, int64_t M, int32_t chunk,
                           const ClusterBufs& b, hipStream_t stream) {
  const int64_t ncl = heads * M;
  if (M <= kMaxBins) {
    const int64_t tiles = (NK + kHistTile - 1) / kHistTile;
    const size_t lds = sizeof(int32_t) * (size_t)M;
    auto big = [&](auto kern) -> hipError_t {
      return lds > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                         : hipSuccess;
    };
    if (big(hist_kernel) != hipSuccess || big(scatter_kernel) != hipSuccess) return hipErrorInvalidValue;
    PISA_LAUNCH("cluster_hist", stream, hist_kernel, dim3((unsigned)tiles, (unsigned)heads), dim3(256), lds, keys, NK,
                M, tiles, b.hist);
    PISA_LAUNCH("cluster_scan", stream, col_scan_kernel, dim3((unsigned)((M + 255) / 256), (unsigned)heads),
                dim3(256), 0, b.hist, M, tiles, b.counts);
    PISA_LAUNCH("cluster_scan", stream, bin_scan_kernel, dim3((unsigned)heads), dim3(1024), 0, b.counts, NK, M,
                b.offsets);
    PISA_LAUNCH("cluster_chunks", stream, chunk_scan_kernel, dim3(1), dim3(1024), 0, b.counts, ncl, chunk,
                b.chunk_off);
    PISA_LAUNCH("cluster_scatter", stream, scatter_kernel, dim3((unsigned)tiles, (unsigned)heads), dim3(256), lds,
                keys, NK, K, M, tiles, b.hist, b.offsets, b.pairs);
    return hipGetLastError();
  }
  const int64_t entries = heads * NK;
  const unsigned ew = (unsigned)((entries + 255) / 256 < 65536 ? (entries + 255) / 256 : 65536);
  const unsigned cw = (unsigned)((ncl + 255) / 256 < 65536 ? (ncl + 255) / 256 : 65536);
  PISA_LAUNCH("cluster_zero", stream, fill_i32_kernel, dim3(cw), dim3(256), 0, b.counts, ncl, 0);
  PISA_LAUNCH("cluster_zero", stream, fill_i32_kernel, dim3(cw), dim3(256), 0, b.cursor, ncl, 0);
  PISA_LAUNCH("cluster_count", stream, atomic_count_kernel, dim3(ew), dim3(256), 0, keys, entries, NK, M, b.counts);
  PISA_LAUNCH("cluster_scan", stream, offset_scan_kernel, dim3(1), dim3(1024), 0, b.counts, ncl, b.offsets);
  PISA_LAUNCH("cluster_chunks", stream, chunk_scan_kernel, dim3(1), dim3(1024), 0, b.counts, ncl, chunk,
              b.chunk_off);
  PISA_LAUNCH("cluster_fill", stream, atomic_fill_kernel, dim3(ew), dim3(256), 0, keys, entries, NK, K, M, b.offsets,
              b.cursor, b.pairs);
  return hipGetLastError();
}

}  // namespace pisa
