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
// MFMA rows = 16 / G_Q queries x G_Q heads (v_mfma_f32_16x16x32_bf16; fp32
// inputs use v_mfma_f32_16x16x4_f32).  The key tile sits in LDS with a
// 16-byte row pad so that the 16 lanes of a fragment read hit distinct banks.
#include "kernels.h"

namespace pisa {

constexpr int kS2Waves = 4;
constexpr int kS2Chunk = 256;  // queries of one cluster per workgroup
constexpr int kTopkWaves = 4;

// ---- workspace layout -------------------------------------------------------
struct S2Layout {
  int64_t ncl;      // clusters = B * Hkv * bins per head
  int64_t max_pairs;
  size_t off_counts, off_cursor, off_offsets, off_chunks, off_pairs, off_scores, off_hist, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static S2Layout s2_layout(const Problem& p) {
  S2Layout s{};
  const int64_t M2 = level_rows(p.N, p.C, 2);
  const int64_t Mb = cluster_bins(p.N, M2, M2);  // (query block, level-2 block) bins per head
  s.ncl = (int64_t)p.B * p.Hkv * Mb;
  s.max_pairs = (int64_t)p.B * p.Hkv * p.N * p.K;
  size_t off = 0;
  s.off_counts = off;
  off = align256(off + sizeof(int32_t) * s.ncl);
  s.off_cursor = off;
  off = align256(off + sizeof(int32_t) * s.ncl);
  s.off_offsets = off;
  off = align256(off + sizeof(int32_t) * (s.ncl + 1));
  s.off_chunks = off;
  off = align256(off + sizeof(int32_t) * (s.ncl + 1));
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
  const int32_t* pairs;
  float* scores;  // [B][Hkv][N][K][2]
  int64_t ncl, M1, M2, Mb;  // Mb: cluster bins per head
  int32_t B, N, Hq, Hkv, C, K;
  int32_t causal;
  int64_t cap;
  float scale;
};

// NCB: 16-key blocks covering the 2C keys of a tile (2C <= 16 NCB).
// CB0: blocks of the first leaf when C is a multiple of 16 (C = 16 CB0), so
// the leaf of a block is known at compile time; 0 for other C.
// Transposed tiles: S^T = K Q^T with the keys as MFMA rows (A from LDS) and
// 16 columns = 16 / G_Q queries x G_Q heads (B = q rows), so the LSE over a
// leaf's keys is an in-lane reduction plus two cross-group shuffles, and the
// GQA sum is a shuffle over the G_Q columns of a query.
template <typename T, int D, int G, int NCB, int CB0>
__global__ __launch_bounds__(kS2Waves* kWave) void leaf_score_kernel(S2Args a) {
  constexpr int NS = D / 32;                  // 32-wide contraction steps
  constexpr int TQ = 16 / G;                  // queries per 16-column tile
  constexpr int PITCH = D + 16 / sizeof(T);   // LDS row pitch (elements)
  constexpr float kLog2e = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* s_k = reinterpret_cast<T*>(smem_raw);  // [NCB*16][PITCH]

  const int64_t chunk = blockIdx.x;
  if (chunk >= a.chunk_off[a.ncl]) return;  // uniform over the workgroup
  // cluster c with chunk_off[c] <= chunk < chunk_off[c + 1]
  int64_t lo = 0, hi = a.ncl;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (a.chunk_off[mid] <= chunk) lo = mid;
    else hi = mid;
  }
  const int64_t c = lo;
  const int64_t bh = c / a.Mb;
  const int64_t j2 = c % a.M2;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int64_t p_begin = a.offsets[c] + (chunk - a.chunk_off[c]) * (int64_t)kS2Chunk;
  const int64_t p_end_c = (int64_t)a.offsets[c] + a.counts[c];
  const int64_t p_end = p_begin + kS2Chunk < p_end_c ? p_begin + kS2Chunk : p_end_c;

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
  __syncthreads();

  const int w = threadIdx.x / kWave, lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const int qi = col / G, hh = col % G;
  const T* qb = static_cast<const T*>(a.q);
  const float sl2 = a.scale * kLog2e;  // logits in log2 units
  float* out_base = a.scores + bh * (int64_t)a.N * a.K * 2;
  auto load_q = [&](int32_t prq, Frag<T>* f) {
    if (prq >= 0) {
      const T* qrow = qb + (((int64_t)b * a.Hq + h * G + hh) * a.N + (prq >> 5)) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) f[s].load(qrow + g * (D / 4) + 8 * s);
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) f[s].zero();
    }
  };
  const int64_t stride = (int64_t)kS2Waves * TQ;
  int64_t tile = p_begin + (int64_t)w * TQ;
  int32_t pr = (tile + qi < p_end) ? a.pairs[tile + qi] : -1;
  Frag<T> fq[NS];
  load_q(pr, fq);
  for (; tile < p_end; tile += stride) {
    // prefetch the next tile's pair and query rows
    const int32_t pr_n = (tile + stride + qi < p_end) ? a.pairs[tile + stride + qi] : -1;
    Frag<T> fn[NS];
    load_q(pr_n, fn);
    // re-read the key fragments from LDS every tile rather than keeping all
    // of them live in registers (which would cap occupancy at one wave): the
    // offset is opaque to the compiler, the pointer stays an LDS pointer
    int koff = 0;
    asm volatile("" : "+v"(koff));
    const T* sk = s_k + koff;
    floatx4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Frag<T> fk;
        fk.load(sk + (cb * 16 + col) * PITCH + g * (D / 4) + 8 * s);
        acc[cb] = mma(fk, fq[s], acc[cb]);
      }
    }
    // keys key_local < lim count for this column's query (t >= key0 + key_local)
    int lim = 0;
    if (pr >= 0) {
      const int64_t t = pr >> 5;
      lim = a.causal ? (int)((t - key0 + 1) < nkeys ? (t - key0 + 1) : nkeys) : nkeys;
    }
    // masked raw dot products (the mask only where some column of the tile
    // sees fewer keys than the tile holds); max per leaf; exp2 of
    // (x - max) * scale*log2e
    if (__ballot(lim < NCB * 16) != 0ull) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cb * 16 + 4 * g + i >= lim) acc[cb][i] = -INFINITY;
    }
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kl = cb * 16 + 4 * g + i;
        const bool first = CB0 ? (cb < CB0) : (kl < C);
        if (first) mx0 = fmaxf(mx0, acc[cb][i]);
        else mx1 = fmaxf(mx1, acc[cb][i]);
      }
    mx0 = fmaxf(mx0, __shfl_xor(mx0, 16));
    mx0 = fmaxf(mx0, __shfl_xor(mx0, 32));
    mx1 = fmaxf(mx1, __shfl_xor(mx1, 16));
    mx1 = fmaxf(mx1, __shfl_xor(mx1, 32));
    const float nb0 = -mx0 * sl2, nb1 = -mx1 * sl2;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kl = cb * 16 + 4 * g + i;
        const bool first = CB0 ? (cb < CB0) : (kl < C);
        if (first) s0 += exp2_nonpos(fmaf(acc[cb][i], sl2, nb0));  // exp2(-inf) = 0
        else s1 += exp2_nonpos(fmaf(acc[cb][i], sl2, nb1));
      }
    s0 += __shfl_xor(s0, 16);
    s0 += __shfl_xor(s0, 32);
    s1 += __shfl_xor(s1, 16);
    s1 += __shfl_xor(s1, 32);
    constexpr float kLn2 = 0.6931471805599453f;
    float u0 = (mx0 == -INFINITY) ? -INFINITY : mx0 * a.scale + __log2f(s0) * kLn2;
    float u1 = (mx1 == -INFINITY) ? -INFINITY : mx1 * a.scale + __log2f(s1) * kLn2;
    // GQA sum over the G columns of the query
    u0 = lane_group_sum<G>(u0);
    u1 = lane_group_sum<G>(u1);
    if (g == 0 && hh == 0 && pr >= 0) {
      const int64_t e = (int64_t)(pr >> 5) * a.K + (pr & 31);  // (t, slot) entry
      out_base[e * 2] = u0;
      out_base[e * 2 + 1] = u1;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) fq[s] = fn[s];
    pr = pr_n;
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
// half sorts, then a K-lane index sort), else 0 (full wave sorts).
template <int KP>
__global__ __launch_bounds__(kTopkWaves* kWave) void final_topk_kernel(TopkArgs a) {
  const int64_t wid = (int64_t)blockIdx.x * kTopkWaves + threadIdx.x / kWave;
  const int64_t total = (int64_t)a.B * a.Hkv * a.N;
  if (wid >= total) return;
  const int lane = lane_id();
  const int slot = lane >> 1, l = lane & 1;
  uint64_t key = 0ull;
  if (slot < a.K) {
    const int32_t j2 = a.blk2[wid * a.K + slot];
    if (j2 >= 0) {
      const float sc = a.scores[(wid * a.K + slot) * 2 + l];
      if (sc != -INFINITY) key = score_key(sc, 2 * j2 + l);
    }
  }
  if (KP) key = top_half<(KP ? KP : 16)>(key);
  else key = wave_sort_desc(key);
  const bool kept = lane < a.K && key != 0ull;
  uint64_t k2 = kept ? index_key(key_index(key), key_score(key)) : 0ull;
  if (KP) k2 = group_sort_desc<(KP ? KP : 16)>(k2);
  else k2 = wave_sort_desc(k2);
  if (lane < a.K) {
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
  int32_t* pairs = reinterpret_cast<int32_t*>(base + L.off_pairs);
  float* scores = reinterpret_cast<float*>(base + L.off_scores);
  const int64_t M1 = level_rows(p.N, p.C, 1), M2 = level_rows(p.N, p.C, 2);
  const int64_t entries = (int64_t)p.B * p.Hkv * p.N * p.K;
  const ClusterBufs cb{counts, cursor, offsets, chunk_off, pairs, reinterpret_cast<int32_t*>(base + L.off_hist)};
  hipError_t err = launch_clusters(blk2, (int64_t)p.B * p.Hkv, (int64_t)p.N * p.K, p.K, M2, M2, kS2Chunk, cb, stream);
  if (err != hipSuccess) return err;
  S2Args a{q, k, counts, offsets, chunk_off, pairs, scores, L.ncl, M1, M2, cluster_bins(p.N, M2, M2), p.B, p.N, p.Hq, p.Hkv,
           p.C, p.K,
           p.causal ? 1 : 0, p.cap, p.scale};
  const int64_t max_chunks = (entries + kS2Chunk - 1) / kS2Chunk + L.ncl;
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
    hipError_t e;
    if (p.C == 32)
      e = run(leaf_score_kernel<T, D, G, 4, 2>);
    else if (p.C == 64)
      e = run(leaf_score_kernel<T, D, G, 8, 4>);
    else if (p.C == 128)
      e = run(leaf_score_kernel<T, D, G, 16, 8>);
    else if (p.C <= 32)
      e = run(leaf_score_kernel<T, D, G, 4, 0>);
    else if (p.C <= 64)
      e = run(leaf_score_kernel<T, D, G, 8, 0>);
    else
      e = run(leaf_score_kernel<T, D, G, 16, 0>);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  });
  if (err != hipSuccess) return err;
  TopkArgs ta{blk2, scores, idx, score, p.B, p.N, p.Hkv, p.K};
  const int64_t waves = (int64_t)p.B * p.Hkv * p.N;
  const dim3 tgrid((unsigned)((waves + kTopkWaves - 1) / kTopkWaves)), tblock(kTopkWaves * kWave);
  if (p.K == 16)
    PISA_LAUNCH("final_topk", stream, final_topk_kernel<16>, tgrid, tblock, 0, ta);
  else if (p.K == 32)
    PISA_LAUNCH("final_topk", stream, final_topk_kernel<32>, tgrid, tblock, 0, ta);
  else
    PISA_LAUNCH("final_topk", stream, final_topk_kernel<0>, tgrid, tblock, 0, ta);
  return hipGetLastError();
}

}  // namespace pisa
