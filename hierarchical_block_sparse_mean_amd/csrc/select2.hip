// Stage 2 of the two-stage selector and the final top-K.
//
// "Block Sparse Attention with Log-Linear Complexity" (PISA), hyper.ai page,
// section "kernel implementation": after stage 1 every query has at most gK
// candidate leaves; queries that must score the same candidate key block are
// grouped into clusters, each cluster is cut into tiles of queries, one
// program loads a key tile once and reuses it for a (Q_tile * G_Q) x d query
// tile (the (Q_tile G_Q) x d times d x C contraction), applies the LSE over
// the keys per query head and sums over the G_Q heads; a last kernel applies
// top-K per (query, KV head).  The leaf score is the exact raw-key LSE
// (section "coarse-to-fine top-K selection", score equation at level 1).
//
// Design on gfx950: a cluster is a kept level-2 block (its two sibling leaves
// are always candidates together), so one key tile of 2C keys serves both
// leaves and each query row is read once per pair of leaves.  Tiles are 16
// MFMA columns = 16 / G_Q queries x G_Q heads (v_mfma_f32_16x16x32_bf16; fp32
// inputs use v_mfma_f32_16x16x4_f32); Q_tile = 16 / G_Q or, taking two tiles
// per key-fragment read, 32 / G_Q.  The key tile sits in LDS with a 16-byte
// row pad so that the 16 lanes of a fragment read hit distinct banks.
#include "kernels.h"

namespace pisa {

constexpr int kS2Waves = 4;
constexpr int kS2Chunk = 1024;  // pairs of one cluster per workgroup (its key tile is staged once per chunk)
constexpr int kTopkWaves = 4;

// ---- workspace layout -------------------------------------------------------
struct S2Layout {
  int64_t ncl;      // clusters = B * Hkv * bins per head
  int64_t max_pairs, max_chunks;
  size_t off_counts, off_cursor, off_offsets, off_chunks, off_map, off_pairs, off_scores, off_hist, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static S2Layout s2_layout(const Problem& p) {
  S2Layout s{};
  const int64_t M2 = level_rows(p.N, p.C, 2);
  const int64_t Mb = cluster_bins(p.N, M2, M2);  // (query block, level-2 block) bins per head
  s.ncl = (int64_t)p.B * p.Hkv * Mb;
  s.max_pairs = (int64_t)p.B * p.Hkv * p.N * p.K;
  s.max_chunks = (s.max_pairs + kS2Chunk - 1) / kS2Chunk + s.ncl;
  size_t off = 0;
  s.off_counts = off;
  off = align256(off + sizeof(int32_t) * s.ncl);
  s.off_cursor = off;
  off = align256(off + sizeof(int32_t) * s.ncl);
  s.off_offsets = off;
  off = align256(off + sizeof(int32_t) * (s.ncl + 1));
  s.off_chunks = off;
  off = align256(off + sizeof(int32_t) * (s.ncl + 1));
  s.off_map = off;
  off = align256(off + sizeof(ChunkEntry) * s.max_chunks);
  s.off_pairs = off;
  off = align256(off + sizeof(int32_t) * s.max_pairs);
  s.off_scores = off;
  off = align256(off + sizeof(float) * 2 * s.max_pairs);
  s.off_hist = off;
  off = align256(off + cluster_scratch_bytes((int64_t)p.B * p.Hkv, (int64_t)p.N * p.K, Mb));
  s.total = off;
  return s;
}

size_t stage2_workspace_bytes(const Problem& p) { return s2_layout(p).total; }

struct S2Args {
  const void* q;
  const void* k;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* chunk_off;
  const ChunkEntry* chunk_map;  // work chunk -> (cluster, first pair, pairs)
  const int32_t* pairs;
  float* scores;  // [B][Hkv][N][K][2]
  int64_t ncl, M1, M2, Mb;  // Mb: cluster bins per head
  int32_t B, N, Hq, Hkv, C, K;
  int32_t causal;
  int64_t cap;
  float scale;
};

// NCB: 16-key blocks covering the 2C keys of a tile (2C <= 16 NCB).
// CB0: blocks of the first leaf when C is a multiple of 16 (C = 16 CB0): the
// two leaves are then scored one after the other, CB0 blocks each; 0 for
// other C (one pass over all NCB blocks, the leaf of a key by its index).
// TT: query tiles scored together, so that each key fragment read from LDS
// feeds TT products (the LDS traffic per pair falls by TT).
// Transposed tiles: S^T = K Q^T with the keys as MFMA rows (A from LDS) and
// 16 columns = 16 / G_Q queries x G_Q heads (B = q rows), so the LSE over a
// leaf's keys is an in-lane reduction plus two cross-group shuffles, and the
// GQA sum is a shuffle over the G_Q columns of a query.
template <typename T, int D, int G, int NCB, int CB0, int TT>
__global__ __launch_bounds__(kS2Waves* kWave) PISA_MFMA_REGS void leaf_score_kernel(S2Args a) {
  constexpr int NS = D / 32;                  // 32-wide contraction steps
  constexpr int TQ = 16 / G;                  // queries per 16-column tile
  constexpr int PITCH = D + 16 / sizeof(T);   // LDS row pitch (elements)
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* s_k = reinterpret_cast<T*>(smem_raw);  // [NCB*16][PITCH]
  __shared__ int32_t s_pr[kS2Chunk];        // the chunk's pair codes

  const ChunkEntry ce = a.chunk_map[blockIdx.x];
  if (ce.cluster < 0) return;  // past the last work chunk (uniform over the workgroup)
  const int64_t c = ce.cluster;
  const int64_t bh = c / a.Mb;
  const int64_t j2 = c % a.M2;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int64_t p_begin = ce.begin;
  const int64_t p_end = p_begin + ce.count;

  // key tile: leaves 2*j2 and 2*j2+1 are the contiguous keys [key0, key0 + 2C)
  const int C = a.C;
  const int rows = 2 * C;
  const T* kh = static_cast<const T*>(a.k) + bh * a.cap * D;
  const int64_t key0 = 2 * j2 * (int64_t)C;
  const int nkeys = (int)((a.N - key0) < rows ? (a.N - key0) : rows);  // existing keys
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  for (int i = threadIdx.x; i < NCB * 16 * (D / EPV); i += blockDim.x) {
    const int r = i / (D / EPV), d = (i % (D / EPV)) * EPV;
    uint4 v = {0u, 0u, 0u, 0u};
    if (r < nkeys) v = *reinterpret_cast<const uint4*>(kh + (key0 + r) * D + d);
    *reinterpret_cast<uint4*>(s_k + r * PITCH + d) = v;
  }
  for (int i = threadIdx.x; i < kS2Chunk; i += blockDim.x)
    s_pr[i] = p_begin + i < p_end ? a.pairs[p_begin + i] : -1;
  __syncthreads();

  const int w = threadIdx.x / kWave, lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const int qi = col / G, hh = col % G;
  const T* qb = static_cast<const T*>(a.q);
  const float sl2 = a.scale * kLog2e;  // logits in log2 units
  float* out_base = a.scores + bh * (int64_t)a.N * a.K * 2;
  // q rows of the column's query; an empty column (prq < 0) reads query 0's
  // rows, finite data whose results are masked and never stored
  auto load_q = [&](int32_t prq, Frag<T>* f) {
    const int64_t tq = prq >= 0 ? (prq >> 5) : 0;
    const T* qrow = qb + (((int64_t)b * a.Hq + h * G + hh) * a.N + tq) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) f[s].load(qrow + 32 * s + 8 * g);
  };
  // keys key_local < limit count for the column's query (t >= key0 + key_local)
  auto limit = [&](int32_t pr) -> int {
    if (pr < 0) return 0;
    const int64_t t = pr >> 5;
    return a.causal ? (int)((t - key0 + 1) < nkeys ? (t - key0 + 1) : nkeys) : nkeys;
  };
  // LSE of one leaf from this lane's (masked) logits: max and sum of exp2 of
  // (x - max) * scale*log2e, each over the lane's values and then the four
  // lane groups (rows of the accumulator tiles)
  auto leaf_lse = [&](float mx, auto&& sum_exp) -> float {
    mx = rows_max(mx);
    const float sm = rows_sum(sum_exp(-mx * sl2));  // exp2(-inf) = 0
    return (mx == -INFINITY) ? -INFINITY : mx * a.scale + __log2f(sm) * kLn2;
  };
  // the two leaf scores of TT tiles of 16 / G_Q pairs each (column query qi)
  auto score_tiles = [&](Frag<T> (&fq)[TT][NS], const int32_t (&pr)[TT], auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    // re-read the key fragments from LDS every step rather than keeping all
    // of them live in registers (which would cap occupancy at one wave): the
    // offset is opaque to the compiler, the pointer stays an LDS pointer
    int koff = 0;
    asm volatile("" : "+v"(koff));
    const T* sk = s_k + koff;
    int lim[TT];
    float u[TT][2];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) lim[tt] = limit(pr[tt]);
    if constexpr (CB0 > 0) {
#pragma unroll
      for (int leaf = 0; leaf < 2; ++leaf) {
        floatx4 acc[TT][CB0];
#pragma unroll
        for (int cb = 0; cb < CB0; ++cb) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) acc[tt][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            Frag<T> fk;
            fk.load(sk + ((leaf * CB0 + cb) * 16 + col) * PITCH + 32 * s + 8 * g);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) acc[tt][cb] = mma(fk, fq[tt][s], acc[tt][cb]);
          }
        }
        // masked chunks: keys at or beyond the column's limit drop out
        if constexpr (MASK) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int cb = 0; cb < CB0; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[tt][cb][i] = (leaf * CB0 + cb) * 16 + 4 * g + i >= lim[tt] ? -INFINITY : acc[tt][cb][i];
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          float mx = -INFINITY;
#pragma unroll
          for (int cb = 0; cb < CB0; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, acc[tt][cb][i]);
          u[tt][leaf] = leaf_lse(mx, [&](float nb) {
            float sm = 0.f;
#pragma unroll
            for (int cb = 0; cb < CB0; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i) sm += exp2_nonpos(fmaf(acc[tt][cb][i], sl2, nb));
            return sm;
          });
        }
      }
    } else {
      floatx4 acc[TT][NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Frag<T> fk;
          fk.load(sk + (cb * 16 + col) * PITCH + 32 * s + 8 * g);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) acc[tt][cb] = mma(fk, fq[tt][s], acc[tt][cb]);
        }
      }
      // (all-zero key rows beyond 2C are masked too)
      bool part = false;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) part |= lim[tt] < NCB * 16;
      if (__ballot(part) != 0ull) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (cb * 16 + 4 * g + i >= lim[tt]) acc[tt][cb][i] = -INFINITY;
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int leaf = 0; leaf < 2; ++leaf) {
          // key kl belongs to leaf (kl >= C)
          float mx = -INFINITY;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((cb * 16 + 4 * g + i >= C) == (leaf == 1)) mx = fmaxf(mx, acc[tt][cb][i]);
          u[tt][leaf] = leaf_lse(mx, [&](float nb) {
            float sm = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if ((cb * 16 + 4 * g + i >= C) == (leaf == 1)) sm += exp2_nonpos(fmaf(acc[tt][cb][i], sl2, nb));
            return sm;
          });
        }
      }
    }
    // GQA sum over the G columns of each query
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float u0 = lane_group_sum<G>(u[tt][0]);
      const float u1 = lane_group_sum<G>(u[tt][1]);
      if (g == 0 && hh == 0 && pr[tt] >= 0) {
        const int64_t e = (int64_t)(pr[tt] >> 5) * a.K + (pr[tt] & 31);  // (t, slot) entry
        // (a streaming store: read once, by the final top-K)
        __builtin_nontemporal_store(floatx2_t{u0, u1}, reinterpret_cast<floatx2_t*>(out_base + e * 2));
      }
    }
  };
  // steps of TT tiles: wave w takes steps w, w + W, w + 2W, ... (W = waves)
  // of the chunk, with two query-row buffers: the next step's rows load
  // while the current step is scored
  constexpr int SP = TT * TQ;  // pairs per step
  const int n = (int)(p_end - p_begin);
  const int stride = kS2Waves * SP;
  auto fetch = [&](int i, int32_t (&pr)[TT], Frag<T> (&f)[TT][NS]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int j = i + tt * TQ + qi;
      pr[tt] = j < n ? s_pr[j] : -1;
      load_q(pr[tt], f[tt]);
    }
  };
  auto run = [&](auto mask_c) {
    Frag<T> fa[TT][NS], fb[TT][NS];
    int32_t pa[TT], pb[TT];
    int i = w * SP;
    if (i >= n) return;
    fetch(i, pa, fa);
    while (true) {
      fetch(i + stride, pb, fb);
      score_tiles(fa, pa, mask_c);
      i += stride;
      if (i >= n) break;
      fetch(i + stride, pa, fa);
      score_tiles(fb, pb, mask_c);
      i += stride;
      if (i >= n) break;
    }
  };
  // With whole leaves (CB0 > 0) the mask is only needed in chunks where some
  // query sees fewer than the 2C keys (its own block under the causal rule,
  // or the last block of the sequence); the rest run without it.
  // Columns without a pair (-1) need no mask: their results are not stored.
  if constexpr (CB0 > 0) {
    bool part = false;
    for (int j = threadIdx.x; j < n; j += blockDim.x) part |= limit(s_pr[j]) < 2 * C;
    if (__syncthreads_or(part)) run(std::true_type{});
    else run(std::false_type{});
  } else {
    run(std::false_type{});
  }
}

// ---- final top-K per (b, h, t) ------------------------------------------------
struct TopkArgs {
  const int32_t* blk2;
  const float* scores;
  int32_t* idx;
  float* score;
  int32_t B, N, Hkv, K;
};

// KP: K when K is 16 or 32 (the 2K candidates sit in lanes [0, 2K): top K by
// half sorts, then a K-lane index sort), else 0 (full wave sorts).  For
// K = 16 a wave takes two (b, h, t) rows, one per 32-lane half (every
// exchange of the half sorts stays inside a half).
template <int KP>
constexpr int topk_rows_per_wave() { return KP == 16 ? 2 : 1; }

template <int KP>
__global__ __launch_bounds__(kTopkWaves* kWave) void final_topk_kernel(TopkArgs a) {
  constexpr int QPW = topk_rows_per_wave<KP>();
  const int lane0 = lane_id();
  const int half = QPW == 2 ? lane0 >> 5 : 0;
  const int lane = QPW == 2 ? lane0 & 31 : lane0;  // lane within the row's lanes
  const int64_t wid0 = ((int64_t)blockIdx.x * kTopkWaves + threadIdx.x / kWave) * QPW;
  const int64_t total = (int64_t)a.B * a.Hkv * a.N;
  if (wid0 >= total) return;  // uniform over the wave
  const int64_t wid = wid0 + half;
  const bool live = wid < total;
  const int slot = lane >> 1, l = lane & 1;
  // the block and its score are loaded together (the score of an empty
  // slot is read but not used), so the row costs one memory round trip
  int32_t j2 = -1;
  float sc = -INFINITY;
  if (live && slot < a.K) {
    j2 = a.blk2[wid * a.K + slot];
    sc = a.scores[(wid * a.K + slot) * 2 + l];
  }
  const uint64_t key0 = (j2 >= 0 && sc != -INFINITY) ? score_key(sc, 2 * j2 + l) : 0ull;
  uint64_t key = key0;
  if (KP) key = top_half<(KP ? KP : 16)>(key);
  else key = wave_sort_desc(key);
  const bool kept = lane < a.K && key != 0ull;
  uint64_t k2 = kept ? index_key(key_index(key), key_score(key)) : 0ull;
  if (KP) k2 = group_sort_desc<(KP ? KP : 16)>(k2);
  else k2 = wave_sort_desc(k2);
  if (live && lane < a.K) {
    const bool v = k2 != 0ull;
    a.idx[wid * a.K + lane] = v ? index_key_index(k2) : -1;
    if (a.score) a.score[wid * a.K + lane] = v ? index_key_score(k2) : -INFINITY;
  }
}

hipError_t launch_stage2(const Problem& p, const void* q, const void* k, const int32_t* blk2, int32_t* idx,
                         float* score, void* ws, hipStream_t stream) {
  const S2Layout L = s2_layout(p);
  char* base = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.off_counts);
  int32_t* cursor = reinterpret_cast<int32_t*>(base + L.off_cursor);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.off_offsets);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + L.off_chunks);
  ChunkEntry* chunk_map = reinterpret_cast<ChunkEntry*>(base + L.off_map);
  int32_t* pairs = reinterpret_cast<int32_t*>(base + L.off_pairs);
  float* scores = reinterpret_cast<float*>(base + L.off_scores);
  const int64_t M1 = level_rows(p.N, p.C, 1), M2 = level_rows(p.N, p.C, 2);
  const int64_t entries = (int64_t)p.B * p.Hkv * p.N * p.K;
  const ClusterBufs cb{counts, cursor, offsets, chunk_off, pairs, reinterpret_cast<int32_t*>(base + L.off_hist)};
  hipError_t err = launch_clusters(blk2, (int64_t)p.B * p.Hkv, (int64_t)p.N * p.K, p.K, M2, M2, kS2Chunk, cb, stream);
  if (err != hipSuccess) return err;
  const int64_t max_chunks = (entries + kS2Chunk - 1) / kS2Chunk + L.ncl;
  err = launch_chunk_map(chunk_off, offsets, counts, L.ncl, kS2Chunk, max_chunks, chunk_map, stream);
  if (err != hipSuccess) return err;
  S2Args a{q, k, counts, offsets, chunk_off, chunk_map, pairs, scores, L.ncl, M1, M2, cluster_bins(p.N, M2, M2), p.B, p.N, p.Hq, p.Hkv,
           p.C, p.K,
           p.causal ? 1 : 0, p.cap, p.scale};
  err = dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    const int ncb = p.C <= 32 ? 4 : (p.C <= 64 ? 8 : 16);
    const size_t lds = (size_t)ncb * 16 * (D + 16 / sizeof(T)) * sizeof(T);
    auto run = [&](auto kern) -> hipError_t {
      if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      PISA_LAUNCH("leaf_score", stream, kern, dim3((unsigned)max_chunks), dim3(kS2Waves * kWave), lds, a);
      return hipSuccess;
    };
    // tiles per step: q_tile / (16 / G_Q), two only for 16-bit inputs with
    // whole 16-key blocks per leaf (fp32 query rows take twice the registers)
    const bool tt2 = sizeof(T) == 2 && p.q_tile * G == 32;
    constexpr int TT2 = sizeof(T) == 2 ? 2 : 1;
    hipError_t e;
    if (p.C == 32)
      e = tt2 ? run(leaf_score_kernel<T, D, G, 4, 2, TT2>) : run(leaf_score_kernel<T, D, G, 4, 2, 1>);
    else if (p.C == 64)
      e = tt2 ? run(leaf_score_kernel<T, D, G, 8, 4, TT2>) : run(leaf_score_kernel<T, D, G, 8, 4, 1>);
    else if (p.C == 128)
      e = tt2 ? run(leaf_score_kernel<T, D, G, 16, 8, TT2>) : run(leaf_score_kernel<T, D, G, 16, 8, 1>);
    else if (p.C <= 32)
      e = run(leaf_score_kernel<T, D, G, 4, 0, 1>);
    else if (p.C <= 64)
      e = run(leaf_score_kernel<T, D, G, 8, 0, 1>);
    else
      e = run(leaf_score_kernel<T, D, G, 16, 0, 1>);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  });
  if (err != hipSuccess) return err;
  TopkArgs ta{blk2, scores, idx, score, p.B, p.N, p.Hkv, p.K};
  const int64_t rows = (int64_t)p.B * p.Hkv * p.N;
  auto grid = [&](int qpw) {
    const int64_t waves = (rows + qpw - 1) / qpw;
    return dim3((unsigned)((waves + kTopkWaves - 1) / kTopkWaves));
  };
  const dim3 tblock(kTopkWaves * kWave);
  if (p.K == 16)
    PISA_LAUNCH("final_topk", stream, final_topk_kernel<16>, grid(topk_rows_per_wave<16>()), tblock, 0, ta);
  else if (p.K == 32)
    PISA_LAUNCH("final_topk", stream, final_topk_kernel<32>, grid(topk_rows_per_wave<32>()), tblock, 0, ta);
  else
    PISA_LAUNCH("final_topk", stream, final_topk_kernel<0>, grid(topk_rows_per_wave<0>()), tblock, 0, ta);
  return hipGetLastError();
}

}  // namespace pisa
