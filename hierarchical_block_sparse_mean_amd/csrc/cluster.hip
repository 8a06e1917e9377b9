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
//      bins gives each bin's first pair; then the work-chunk counts are
//      scanned per head, over the head totals, and the head bases added back;
//   3. per tile, an LDS cursor per bin scatters the pair code (t << 5) | slot.
// A cluster is the set of entries of one (head, query block, key block): the
// queries of a head are cut into blocks of 2^s consecutive positions (the
// smallest s >= 12 whose bins stay within the caller's bin budget, itself at
// most what the LDS histogram holds), so that the work on one block of
// queries is grouped together and the consumers' re-reads of those queries'
// rows stay cache-resident; a budget of M bins keeps one query block.  Bins
// per head: Mb = blocks * M, bin = (t >> s) * M + key block.  Heads with more
// key blocks than the LDS histogram holds use one query block and a
// global-atomic fallback.  Either way: counts[c], offsets[c] (first pair) and
// chunk_off[c] (first work chunk, chunk_off[ncl] = total) for
// c = head * Mb + bin.
//
// Sibling pairing (attention only): an entry's key block is its leaf j,
// except that an even leaf whose odd sibling is the row's next entry (rows
// are ascending) becomes key block M_1 + j / 2, the level-2 block of both,
// and the odd sibling's entry is dropped; the consumer attends both leaves
// of such a block in one tile.
#include "kernels.h"

namespace pisa {

constexpr int kHistTile = 8192;     // entries per histogram tile
constexpr int64_t kMaxBins = kClusterLdsBins;

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

int32_t cluster_query_shift(int64_t N, int64_t M, int64_t max_bins) {
  if (max_bins > kMaxBins) max_bins = kMaxBins;
  if (M >= max_bins) return 31;
  int32_t sh = 12;
  while (sh < 31 && ((N + ((int64_t)1 << sh) - 1) >> sh) * M > max_bins) ++sh;
  return sh;
}

int64_t cluster_bins(int64_t N, int64_t M, int64_t max_bins) {
  const int32_t sh = cluster_query_shift(N, M, max_bins);
  return ((N + ((int64_t)1 << sh) - 1) >> sh) * M;
}

size_t cluster_scratch_bytes(int64_t heads, int64_t NK, int64_t Mb) {
  if (Mb > kMaxBins) return 256;
  const int64_t tiles = (NK + kHistTile - 1) / kHistTile;
  return al256(sizeof(int32_t) * (size_t)heads * tiles * Mb);
}

// bin of entry e_loc = t * K + slot of a head holding key block j, or -1
__device__ __forceinline__ int64_t bin_of(int32_t j, int64_t e_loc, int32_t K, int64_t M, int32_t qshift) {
  if (j < 0 || j >= M) return -1;
  return ((e_loc / K) >> qshift) * M + j;
}

// key block of entry e (e_loc = t * K + slot within its head): keys[e], or
// with sibling pairing (pair_m1 = M_1 > 0) the level-2 block M_1 + j / 2 for
// an even leaf j followed by j + 1, and -1 for that odd sibling
__device__ __forceinline__ int32_t entry_key(const int32_t* __restrict__ keys, int64_t e, int64_t e_loc, int32_t K,
                                             int64_t pair_m1) {
  int32_t j = keys[e];
  if (pair_m1 > 0 && j >= 0) {
    if (j >= pair_m1) return -1;  // not a leaf
    const int32_t slot = (int32_t)(e_loc % K);
    if ((j & 1) == 0) {
      if (slot + 1 < K && j + 1 < pair_m1 && keys[e + 1] == j + 1) j = (int32_t)pair_m1 + (j >> 1);
    } else if (slot > 0 && keys[e - 1] == j - 1) {
      j = -1;
    }
  }
  return j;
}

__global__ void hist_kernel(const int32_t* __restrict__ keys, int64_t NK, int32_t K, int64_t M, int64_t pair_m1,
                            int32_t qshift, int64_t Mb, int64_t tiles, int32_t* __restrict__ hist) {
  extern __shared__ int32_t s_h[];
  const int64_t head = blockIdx.y, tile = blockIdx.x;
  for (int64_t i = threadIdx.x; i < Mb; i += blockDim.x) s_h[i] = 0;
  __syncthreads();
  const int64_t lo = head * NK + tile * kHistTile;
  const int64_t hi = (tile + 1) * kHistTile < NK ? lo + kHistTile : head * NK + NK;
  for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x) {
    const int64_t el = e - head * NK;
    const int64_t bin = bin_of(entry_key(keys, e, el, K, pair_m1), el, K, M, qshift);
    if (bin >= 0) atomicAdd(&s_h[bin], 1);
  }
  __syncthreads();
  int32_t* out = hist + (head * tiles + tile) * Mb;
  for (int64_t i = threadIdx.x; i < Mb; i += blockDim.x) out[i] = s_h[i];
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

__global__ void scatter_kernel(const int32_t* __restrict__ keys, int64_t NK, int32_t K, int64_t M, int64_t pair_m1,
                               int32_t qshift, int64_t Mb, int64_t tiles, const int32_t* __restrict__ base,
                               const int32_t* __restrict__ offsets, int32_t* __restrict__ pairs) {
  extern __shared__ int32_t s_cur[];
  const int64_t head = blockIdx.y, tile = blockIdx.x;
  const int32_t* b = base + (head * tiles + tile) * Mb;
  for (int64_t i = threadIdx.x; i < Mb; i += blockDim.x) s_cur[i] = offsets[head * Mb + i] + b[i];
  __syncthreads();
  const int64_t lo = head * NK + tile * kHistTile;
  const int64_t hi = (tile + 1) * kHistTile < NK ? lo + kHistTile : head * NK + NK;
  for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x) {
    const int64_t el = e - head * NK;
    const int64_t bin = bin_of(entry_key(keys, e, el, K, pair_m1), el, K, M, qshift);
    if (bin >= 0) pairs[atomicAdd(&s_cur[bin], 1)] = pair_code(el, K);
  }
}

// Exclusive scan of the work-chunk counts of all clusters, in three steps:
// per head (one workgroup each) over its Mb bins, over the head totals, and
// the head bases added back.  head_tot: one int per head (scratch).
__global__ __launch_bounds__(1024) void chunk_scan_kernel(const int32_t* __restrict__ counts, int64_t Mb,
                                                          int32_t chunk, int32_t* chunk_off, int32_t* head_tot) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_carry;
  const int64_t head = blockIdx.x;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < Mb; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int32_t v = i < Mb ? (counts[head * Mb + i] + chunk - 1) / chunk : 0;
    s_part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? s_part[threadIdx.x - o] : 0;
      __syncthreads();
      s_part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < Mb) chunk_off[head * Mb + i] = s_carry + s_part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry += s_part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) head_tot[head] = s_carry;
}

// Exclusive scan of the head totals (in place), total into chunk_off[ncl].
__global__ __launch_bounds__(1024) void head_scan_kernel(int32_t* head_tot, int64_t heads, int32_t* chunk_off,
                                                         int64_t ncl) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < heads; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int32_t v = i < heads ? head_tot[i] : 0;
    s_part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? s_part[threadIdx.x - o] : 0;
      __syncthreads();
      s_part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < heads) head_tot[i] = s_carry + s_part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry += s_part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) chunk_off[ncl] = s_carry;
}

__global__ void head_base_kernel(int32_t* chunk_off, const int32_t* __restrict__ head_base, int64_t Mb, int64_t ncl) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < ncl; i += (int64_t)gridDim.x * blockDim.x)
    chunk_off[i] += head_base[i / Mb];
}

// ---- fallback for heads with more than kMaxBins key blocks ----------------------
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void atomic_count_kernel(const int32_t* __restrict__ keys, int64_t entries, int64_t NK, int32_t K,
                                    int64_t M, int64_t pair_m1, int32_t qshift, int64_t Mb, int32_t* counts) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < entries;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bin = bin_of(entry_key(keys, e, e % NK, K, pair_m1), e % NK, K, M, qshift);
    if (bin >= 0) atomicAdd(&counts[(e / NK) * Mb + bin], 1);
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
                                   int64_t M, int64_t pair_m1, int32_t qshift, int64_t Mb,
                                   const int32_t* __restrict__ offsets, int32_t* cursor, int32_t* pairs) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < entries;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bin = bin_of(entry_key(keys, e, e % NK, K, pair_m1), e % NK, K, M, qshift);
    if (bin < 0) continue;
    const int64_t c = (e / NK) * Mb + bin;
    pairs[offsets[c] + atomicAdd(&cursor[c], 1)] = pair_code(e % NK, K);
  }
}

// chunk_off[c] for every cluster (counts known): see chunk_scan_kernel
static hipError_t launch_chunk_scan(const ClusterBufs& b, int64_t heads, int64_t Mb, int32_t chunk,
                                    hipStream_t stream) {
  const int64_t ncl = heads * Mb;
  PISA_LAUNCH("cluster_chunks", stream, chunk_scan_kernel, dim3((unsigned)heads), dim3(1024), 0, b.counts, Mb, chunk,
              b.chunk_off, b.cursor);
  PISA_LAUNCH("cluster_chunks", stream, head_scan_kernel, dim3(1), dim3(1024), 0, b.cursor, heads, b.chunk_off, ncl);
  const unsigned blocks = (unsigned)((ncl + 255) / 256 < 65536 ? (ncl + 255) / 256 : 65536);
  PISA_LAUNCH("cluster_chunks", stream, head_base_kernel, dim3(blocks), dim3(256), 0, b.chunk_off, b.cursor, Mb, ncl);
  return hipGetLastError();
}

// map[ch] = (c, first pair, pairs) for every work chunk ch of cluster c, and
// cluster -1 for ch from chunk_off[ncl] to max_chunks: the consumers' first
// and only lookup (they used to read the chunk total, the cluster, and then
// its offset and count, three dependent loads before any work)
__global__ void chunk_map_kernel(const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ offsets,
                                 const int32_t* __restrict__ counts, int64_t ncl, int32_t chunk, int64_t max_chunks,
                                 ChunkEntry* __restrict__ map) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (int64_t c = tid; c < ncl; c += stride) {
    const int32_t lo = chunk_off[c], hi = chunk_off[c + 1];
    const int32_t off = offsets[c], cnt = counts[c];
    for (int32_t ch = lo; ch < hi; ++ch) {
      const int32_t first = (ch - lo) * chunk;
      const int32_t rest = cnt - first;
      map[ch] = ChunkEntry{(int32_t)c, off + first, rest < chunk ? rest : chunk, 0};
    }
  }
  for (int64_t ch = chunk_off[ncl] + tid; ch < max_chunks; ch += stride) map[ch] = ChunkEntry{-1, 0, 0, 0};
}

hipError_t launch_chunk_map(const int32_t* chunk_off, const int32_t* offsets, const int32_t* counts, int64_t ncl,
                            int32_t chunk, int64_t max_chunks, ChunkEntry* map, hipStream_t stream) {
  const int64_t work = ncl > max_chunks ? ncl : max_chunks;
  const unsigned blocks = (unsigned)((work + 255) / 256 < 65536 ? (work + 255) / 256 : 65536);
  PISA_LAUNCH("cluster_chunks", stream, chunk_map_kernel, dim3(blocks), dim3(256), 0, chunk_off, offsets, counts, ncl,
              chunk, max_chunks, map);
  return hipGetLastError();
}

hipError_t launch_clusters(const int32_t* keys, int64_t heads, int64_t NK, int32_t K, int64_t M, int64_t max_bins,
                           int32_t chunk, const ClusterBufs& b, hipStream_t stream, int64_t pair_m1) {
  const int64_t N = NK / K;
  const int32_t qs = cluster_query_shift(N, M, max_bins);
  const int64_t Mb = cluster_bins(N, M, max_bins);
  const int64_t ncl = heads * Mb;
  if (Mb <= kMaxBins) {
    const int64_t tiles = (NK + kHistTile - 1) / kHistTile;
    const size_t lds = sizeof(int32_t) * (size_t)Mb;
    auto big = [&](auto kern) -> hipError_t {
      return lds > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                         : hipSuccess;
    };
    if (big(hist_kernel) != hipSuccess || big(scatter_kernel) != hipSuccess) return hipErrorInvalidValue;
    PISA_LAUNCH("cluster_hist", stream, hist_kernel, dim3((unsigned)tiles, (unsigned)heads), dim3(256), lds, keys, NK,
                K, M, pair_m1, qs, Mb, tiles, b.hist);
    PISA_LAUNCH("cluster_scan", stream, col_scan_kernel, dim3((unsigned)((Mb + 255) / 256), (unsigned)heads),
                dim3(256), 0, b.hist, Mb, tiles, b.counts);
    PISA_LAUNCH("cluster_scan", stream, bin_scan_kernel, dim3((unsigned)heads), dim3(1024), 0, b.counts, NK, Mb,
                b.offsets);
    if (launch_chunk_scan(b, heads, Mb, chunk, stream) != hipSuccess) return hipGetLastError();
    PISA_LAUNCH("cluster_scatter", stream, scatter_kernel, dim3((unsigned)tiles, (unsigned)heads), dim3(256), lds,
                keys, NK, K, M, pair_m1, qs, Mb, tiles, b.hist, b.offsets, b.pairs);
    return hipGetLastError();
  }
  const int64_t entries = heads * NK;
  const unsigned ew = (unsigned)((entries + 255) / 256 < 65536 ? (entries + 255) / 256 : 65536);
  const unsigned cw = (unsigned)((ncl + 255) / 256 < 65536 ? (ncl + 255) / 256 : 65536);
  PISA_LAUNCH("cluster_zero", stream, fill_i32_kernel, dim3(cw), dim3(256), 0, b.counts, ncl, 0);
  PISA_LAUNCH("cluster_count", stream, atomic_count_kernel, dim3(ew), dim3(256), 0, keys, entries, NK, K, M, pair_m1,
              qs, Mb, b.counts);
  PISA_LAUNCH("cluster_scan", stream, offset_scan_kernel, dim3(1), dim3(1024), 0, b.counts, ncl, b.offsets);
  if (launch_chunk_scan(b, heads, Mb, chunk, stream) != hipSuccess) return hipGetLastError();  // cursor as scratch
  PISA_LAUNCH("cluster_zero", stream, fill_i32_kernel, dim3(cw), dim3(256), 0, b.cursor, ncl, 0);
  PISA_LAUNCH("cluster_fill", stream, atomic_fill_kernel, dim3(ew), dim3(256), 0, keys, entries, NK, K, M, pair_m1,
              qs, Mb, b.offsets, b.cursor, b.pairs);
  return hipGetLastError();
}

}  // namespace pisa
