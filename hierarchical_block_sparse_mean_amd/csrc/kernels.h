// Host-side launchers of the PISA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"

namespace pisa {

// Optional per-kernel timing: when enabled (pisa_timer_enable), every launch
// made through PISA_LAUNCH is bracketed by two HIP events recorded on the
// launch stream.
void timer_begin(const char* name, hipStream_t stream);
void timer_end(const char* name, hipStream_t stream);
#define PISA_LAUNCH(name, stream, kernel, grid, block, lds, ...)                  \
  do {                                                                          \
    ::pisa::timer_begin(name, stream);                                          \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);          \
    ::pisa::timer_end(name, stream);                                            \
  } while (0)

// A validated problem (see pisa.h for the meaning of each field).
struct Problem {
  int32_t B, N, Hq, Hkv, G, D, C, K;
  bool causal;
  int32_t dtype;  // 0 fp32, 1 bf16
  float scale;
  int64_t cap;     // k/v row stride in tokens and pyramid capacity
  int32_t L;       // levels of N tokens
  int32_t q_tile;  // stage-2 queries per MFMA tile
  PyrGeom geo;
};

// Calls fn(T*, integral_constant<D>, integral_constant<G>) for the runtime
// dtype / head dim / group size.  Returns hipErrorInvalidValue if unsupported.
template <typename Fn>
hipError_t dispatch_tdg(int32_t dtype, int32_t D, int32_t G, Fn&& fn) {
  auto with_g = [&](auto tp, auto dc) -> hipError_t {
    switch (G) {
      case 1: return fn(tp, dc, std::integral_constant<int, 1>{});
      case 2: return fn(tp, dc, std::integral_constant<int, 2>{});
      case 4: return fn(tp, dc, std::integral_constant<int, 4>{});
      case 8: return fn(tp, dc, std::integral_constant<int, 8>{});
      case 16: return fn(tp, dc, std::integral_constant<int, 16>{});
      default: return hipErrorInvalidValue;
    }
  };
  auto with_d = [&](auto tp) -> hipError_t {
    switch (D) {
      case 64: return with_g(tp, std::integral_constant<int, 64>{});
      case 128: return with_g(tp, std::integral_constant<int, 128>{});
      default: return hipErrorInvalidValue;
    }
  };
  if (dtype == 1) return with_d(static_cast<uint16_t*>(nullptr));
  return with_d(static_cast<float*>(nullptr));
}

// pyramid.hip
hipError_t launch_build_pyramid(const Problem& p, const void* k, float* pyr, hipStream_t stream);

// route.hip: one wave per (b, h, t); fused = all levels incl. raw-key leaves
// (writes idx/score), else stage 1 (writes the kept level-2 blocks to idx).
hipError_t launch_route(const Problem& p, const void* q, const void* k, const float* pyr, int32_t* idx,
                        float* score, bool fused, hipStream_t stream, unsigned long long* counts = nullptr);
// route.hip: query-major attention, one wave per (b, h, t)
hipError_t launch_attn_query(const Problem& p, const void* q, const void* k, const void* v, const int32_t* idx,
                             void* o, float* lse, hipStream_t stream);

// select2.hip: stage 2 (query clusters, MFMA leaf scoring) and final top-K
size_t stage2_workspace_bytes(const Problem& p);
hipError_t launch_stage2(const Problem& p, const void* q, const void* k, const int32_t* blk2, int32_t* idx,
                         float* score, void* ws, hipStream_t stream);

// cluster.hip: entries keys[head * NK + e] in [0, M) (or -1) -> per cluster
// c = head * M + j: counts[c], offsets[c] (first pair; pairs hold e = t*K +
// slot), chunk_off[c] (first work chunk of `chunk` pairs; chunk_off[ncl] is
// the total).  cursor: ncl int32; hist: cluster_scratch_bytes() bytes.
struct ClusterBufs {
  int32_t* counts;
  int32_t* cursor;
  int32_t* offsets;
  int32_t* chunk_off;
  int32_t* pairs;
  int32_t* hist;
};
// Bins per head that the counting sort's LDS histogram holds (64 KB); a head
// with more bins takes the global-atomic path
constexpr int64_t kClusterLdsBins = 16384;
// Bins per head of a clustering of N queries over M key blocks: query blocks
// of 2^cluster_query_shift(N, M, max_bins) positions times M (see cluster.hip).
// max_bins: the clustering's bin budget per head (query blocks are added
// while bins stay within it; M >= max_bins gives one query block).
int32_t cluster_query_shift(int64_t N, int64_t M, int64_t max_bins);
int64_t cluster_bins(int64_t N, int64_t M, int64_t max_bins);
size_t cluster_scratch_bytes(int64_t heads, int64_t NK, int64_t Mb);
// keys: [heads][N][K] block indices (-1 = none), NK = N * K.  pairs holds,
// per cluster c = head * Mb + (t >> shift) * M + block, the codes
// (t << 5) | slot of its entries; the key block of cluster c is c % M.
// pair_m1 > 0 (= M_1, ascending leaf rows, M = M_1 + ceil(M_1 / 2)): an even
// leaf j kept together with j + 1 goes to key block M_1 + j / 2 under the
// slot of j, and the entry of j + 1 is dropped.
hipError_t launch_clusters(const int32_t* keys, int64_t heads, int64_t NK, int32_t K, int64_t M, int64_t max_bins,
                           int32_t chunk, const ClusterBufs& b, hipStream_t stream, int64_t pair_m1 = 0);
// One entry per work chunk: its cluster, first pair and pair count, so a
// workgroup finds its work with one load.  Entries past the last chunk
// (up to max_chunks, the launch grid) hold cluster -1.
struct ChunkEntry {
  int32_t cluster, begin, count, pad;
};
// map[ch] for ch < max_chunks, from the clusters' chunk_off, offsets, counts
// and the pairs per work chunk
hipError_t launch_chunk_map(const int32_t* chunk_off, const int32_t* offsets, const int32_t* counts, int64_t ncl,
                            int32_t chunk, int64_t max_chunks, ChunkEntry* map, hipStream_t stream);

// Attention clusters (forward and backward): (query block, key block) bins
// per head (key blocks: the leaves, and in the forward also the level-2
// blocks of sibling pairs wherever 2C keys fit one tile: C <= 64, or
// C <= 128 for 16-bit inputs, except fp32 rows of d = 128), so one block of
// queries is attended together and its query rows are re-read from cache.
constexpr int64_t kAttnBins = 8192;

// attn_leaf.hip: leaf-major MFMA attention with a merge pass
size_t attn_leaf_workspace_bytes(const Problem& p);
hipError_t launch_attn_leaf(const Problem& p, const void* q, const void* k, const void* v, const int32_t* idx,
                            void* o, float* lse, void* ws, hipStream_t stream);

// attn_bwd.hip: leaf-major backward of the sparse attention
size_t attn_bwd_workspace_bytes(const Problem& p);
hipError_t launch_attn_bwd(const Problem& p, const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           hipStream_t stream);

// flat.hip
hipError_t launch_flat(const Problem& p, const void* q, const float* pyr, int32_t* idx, float* score,
                       hipStream_t stream);

// decode.hip
struct DecodeArgs {
  int32_t S, Hq, Hkv, G, D, C, K, dtype;
  int64_t cap;
  float scale;
  PyrGeom geo;
};
hipError_t launch_decode(const DecodeArgs& a, void* k_cache, void* v_cache, float* pyr, int32_t* len,
                         const void* q_new, const void* k_new, const void* v_new, void* o, int32_t* idx,
                         float* score, int32_t* err, hipStream_t stream);

}  // namespace pisa
