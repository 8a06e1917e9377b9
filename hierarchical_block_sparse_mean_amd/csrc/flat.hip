// Flat single-level block selector, the measurement baseline: every valid
// leaf summary is scored for every query and the top K are kept
// ("Block Sparse Attention with Log-Linear Complexity", hyper.ai page, section
// "block-sparse attention": flat selection scores all ceil(N/C) block
// summaries per query).  Score of leaf j for KV head h at query t:
// sum over the G_Q query heads of q . P_1[j] * scale, computed as
// (sum of the group's queries) . P_1[j] * scale.
#include "kernels.h"
#include "route.h"

namespace pisa {

constexpr int kFlatWaves = 4;

struct FlatArgs {
  const void* q;
  const float* pyr;
  int32_t* idx;
  float* score;
  int32_t B, N, Hq, Hkv, C, K;
  int32_t causal;
  float scale;
  PyrGeom geo;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kFlatWaves* kWave) void flat_kernel(FlatArgs a) {
  __shared__ float s_q[kFlatWaves][D];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % a.Hkv);
  const int64_t r = bid / a.Hkv;
  const int b = (int)(r % a.B);
  const int64_t t = (r / a.B) * kFlatWaves + w;
  if (t >= a.N) return;
  const T* qb = static_cast<const T*>(a.q);
  for (int d = lane; d < D; d += kWave) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) s += load1<T>(qb + (((int64_t)b * a.Hq + h * G + g) * a.N + t) * D + d);
    s_q[w][d] = s;
  }
  wave_sync();
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const float* leaves = a.pyr + (bh * a.geo.rows + a.geo.level_off[1]) * D;
  const int64_t M1 = level_rows(a.N, a.C, 1);
  const int64_t nl = a.causal ? (t / a.C + 1 < M1 ? t / a.C + 1 : M1) : M1;
  uint64_t best = 0ull;  // running top 64, sorted descending across lanes
  for (int64_t base = 0; base < nl; base += kWave) {
    const int64_t j = base + lane;
    uint64_t key = 0ull;
    if (j < nl) {
      float acc[1];
      dots_summary<D, 1>(leaves + j * D, s_q[w], acc);
      key = score_key(acc[0] * a.scale, (int32_t)j);
    }
    key = wave_sort_desc(key);
    // the larger half of two sorted runs is bitonic; merge it descending
    const uint64_t rev = shfl_xor_u64(key, 63);
    uint64_t m = best > rev ? best : rev;
#pragma unroll
    for (int jj = kWave / 2; jj > 0; jj >>= 1) {
      const uint64_t o = shfl_xor_u64(m, jj);
      m = ((lane & jj) == 0) ? (m > o ? m : o) : (m < o ? m : o);
    }
    best = m;
  }
  const bool kept = lane < a.K && best != 0ull;
  uint64_t k2 = kept ? index_key(key_index(best), key_score(best)) : 0ull;
  k2 = wave_sort_desc(k2);
  if (lane < a.K) {
    const bool v = k2 != 0ull;
    const int64_t o = (bh * a.N + t) * a.K + lane;
    a.idx[o] = v ? index_key_index(k2) : -1;
    if (a.score) a.score[o] = v ? index_key_score(k2) : -INFINITY;
  }
}

// ---- MFMA flat selector (bf16 inputs) -------------------------------------------
// A workgroup takes 64 consecutive queries of one KV head, 16 per wave; one
// MFMA column per query holds the group's summed query (the group sum applied
// to q first).  Leaf summaries stream through LDS in tiles of 64 rows from the
// pyramid's block-floating-point fp16 copy (as in stage 1) and are shared by
// the four waves: (16 leaves) x d x (16 queries) fp16 tiles.  Each query keeps
// its candidates in an LDS buffer: a score enters only if it beats the
// current K-th key, and the buffer is compacted (wave sort, keep K) before it
// can overflow.  The kept leaves' scores are then recomputed in fp32 from the
// fp32 summaries and the bf16 queries.
struct FlatMArgs {
  const uint16_t* q;
  const float* pyr;
  const _Float16* f16;
  const int32_t* ex;
  int32_t* idx;
  float* score;
  int32_t B, N, Hq, Hkv, C, K;
  int32_t causal;
  float scale;
  PyrGeom geo;
};

constexpr int kFlatTile = 64;  // leaf rows per LDS tile
constexpr int kFlatCap = 64;   // candidate buffer per query

template <int D, int G>
__global__ __launch_bounds__(kFlatWaves* kWave) PISA_MFMA_REGS void flat_mfma_kernel(FlatMArgs a) {
  constexpr int NS = D / 32;
  constexpr int RP = D + 8;  // fp16 row pitch in LDS
  __shared__ __align__(16) _Float16 s_tile[kFlatTile * RP];
  __shared__ int32_t s_ex[kFlatTile];
  __shared__ uint64_t s_buf[kFlatWaves][16][kFlatCap];
  __shared__ int32_t s_cnt[kFlatWaves][16];
  __shared__ uint64_t s_thr[kFlatWaves][16];
  __shared__ __align__(16) float s_qs[kFlatWaves][D];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int64_t t0 = (int64_t)blockIdx.x * (kFlatWaves * 16);
  const int64_t tw = t0 + w * 16;  // first query of this wave
  const int64_t tq = tw + col;
  const bool qlive = tq < a.N;
  // summed query of column col, contraction elements g*(D/4) + 8st + e
  float qv[NS][8];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[st][e] = 0.f;
  if (qlive) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const uint16_t* qrow = a.q + (((int64_t)b * a.Hq + h * G + gg) * a.N + tq) * D;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        float x[8];
        load8<uint16_t>(qrow + g * (D / 4) + 8 * st, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[st][e] += x[e];
      }
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qv[st][e]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const int eq = row_exponent(mx);
  halfx8 fq[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) fq[st][e] = to_f16_scaled(qv[st][e], eq);

  const _Float16* hb = a.f16 + (bh * a.geo.rows + a.geo.level_off[1]) * D;
  const int32_t* xb = a.ex + bh * a.geo.rows + a.geo.level_off[1];
  const int32_t M1 = (int32_t)level_rows(a.N, a.C, 1);
  auto limit = [&](int64_t t) -> int32_t {  // valid leaves of query t
    if (!a.causal) return M1;
    const int64_t l = t / a.C + 1;
    return (int32_t)(l < M1 ? l : M1);
  };
  const int64_t tlast_b = (t0 + kFlatWaves * 16 - 1 < a.N) ? t0 + kFlatWaves * 16 - 1 : a.N - 1;
  const int32_t nl = limit(tlast_b);                                           // rows the workgroup needs
  const int32_t nlw = tw < a.N ? limit(tw + 15 < a.N ? tw + 15 : a.N - 1) : 0;  // rows this wave needs
  const int32_t lq = qlive ? limit(tq) : 0;
  if (lane < 16) {
    s_cnt[w][lane] = 0;
    s_thr[w][lane] = 0ull;
  }
  const float scale = a.scale;
  for (int32_t base = 0; base < nl; base += kFlatTile) {
    __syncthreads();  // the previous tile is consumed
    constexpr int CH = D / 8;  // 16-byte pieces per row
    for (int i = threadIdx.x; i < kFlatTile * CH; i += kFlatWaves * kWave) {
      const int r = i / CH, piece = i % CH;
      uint4 v = {0u, 0u, 0u, 0u};
      if (base + r < nl) v = *reinterpret_cast<const uint4*>(hb + (int64_t)(base + r) * D + piece * 8);
      *reinterpret_cast<uint4*>(s_tile + r * RP + piece * 8) = v;
    }
    if (threadIdx.x < kFlatTile) s_ex[threadIdx.x] = base + (int)threadIdx.x < nl ? xb[base + threadIdx.x] : 0;
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kFlatTile / 16; ++rb) {
      const int32_t row0 = base + rb * 16;
      if (row0 >= nlw) break;  // wave-uniform
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const halfx8 fa = *reinterpret_cast<const halfx8*>(s_tile + (rb * 16 + col) * RP + g * (D / 4) + 8 * st);
        acc = mma16x16x32(fa, fq[st], acc);
      }
      // lane (g, col): leaves row0 + 4g + i for query col
      const uint64_t thr = s_thr[w][col];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t leaf = row0 + 4 * g + i;
        const float u = ldexpf(acc[i], s_ex[rb * 16 + 4 * g + i] + eq) * scale;
        const uint64_t key = leaf < lq ? score_key(u, leaf) : 0ull;
        if (key > thr) {
          const int pos = atomicAdd(&s_cnt[w][col], 1);
          s_buf[w][col][pos] = key;
        }
      }
      wave_sync();
      // compact the buffers that could overflow on the next 16 leaves
      uint64_t full = __ballot(lane < 16 && s_cnt[w][lane] > kFlatCap - 16);
      while (full) {
        const int qq = __ffsll((long long)full) - 1;
        full &= full - 1;
        const int cnt = s_cnt[w][qq];
        uint64_t k2 = lane < cnt ? s_buf[w][qq][lane] : 0ull;
        k2 = wave_sort_desc(k2);
        const uint64_t kth = (uint64_t)(uint32_t)__shfl((int)(uint32_t)k2, a.K - 1) |
                             ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(k2 >> 32), a.K - 1) << 32);
        wave_sync();
        s_buf[w][qq][lane] = lane < a.K ? k2 : 0ull;
        if (lane == 0) {
          s_cnt[w][qq] = a.K;
          s_thr[w][qq] = kth;
        }
        wave_sync();
      }
    }
  }
  // final top K of each query, in ascending leaf order, with exact scores:
  // lane = (slot, quarter of the dims); the summed query passes through LDS
  const int64_t base_p = bh * a.geo.rows + a.geo.level_off[1];
  for (int qq = 0; qq < 16; ++qq) {
    const int64_t tt = tw + qq;
    if (tt >= a.N) break;  // wave-uniform
    const int cnt = s_cnt[w][qq];
    uint64_t k2 = lane < cnt ? s_buf[w][qq][lane] : 0ull;
    k2 = wave_sort_desc(k2);
    const bool kept = lane < a.K && k2 != 0ull;
    uint64_t k3 = kept ? index_key(key_index(k2), key_score(k2)) : 0ull;
    k3 = wave_sort_desc(k3);
    const int32_t leaf = k3 != 0ull ? index_key_index(k3) : -1;  // lanes < K
    if (col == qq)
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_qs[w][g * (D / 4) + 8 * st + e] = qv[st][e];
    wave_sync();
    for (int s0 = 0; s0 < a.K; s0 += kWave / 4) {
      const int slot = s0 + lane / 4, quarter = lane % 4;
      const int32_t lf = __shfl(leaf, slot < kWave ? slot : 0);
      float dot = 0.f;
      if (slot < a.K && lf >= 0) {
        const float* prow = a.pyr + (base_p + lf) * D + quarter * (D / 4);
        const float* qs = &s_qs[w][quarter * (D / 4)];
#pragma unroll
        for (int d = 0; d < D / 4; d += 4) {
          const float4 pv = *reinterpret_cast<const float4*>(prow + d);
          const float4 qv4 = *reinterpret_cast<const float4*>(qs + d);
          dot = fmaf(pv.x, qv4.x, dot);
          dot = fmaf(pv.y, qv4.y, dot);
          dot = fmaf(pv.z, qv4.z, dot);
          dot = fmaf(pv.w, qv4.w, dot);
        }
      }
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      if (quarter == 0 && slot < a.K) {
        const int64_t o = (bh * a.N + tt) * a.K + slot;
        a.idx[o] = lf;
        if (a.score) a.score[o] = lf >= 0 ? dot * scale : -INFINITY;
      }
    }
    wave_sync();
  }
}

hipError_t launch_flat(const Problem& p, const void* q, const float* pyr, int32_t* idx, float* score,
                       hipStream_t stream) {
  FlatArgs a{q, pyr, idx, score, p.B, p.N, p.Hq, p.Hkv, p.C, p.K, p.causal ? 1 : 0, p.scale, p.geo};
  const int64_t blocks = (int64_t)p.B * p.Hkv * ((p.N + kFlatWaves - 1) / kFlatWaves);
  const int64_t plane = (int64_t)p.B * p.Hkv * p.geo.rows * p.D;
  const _Float16* f16 = reinterpret_cast<const _Float16*>(pyr + plane);
  FlatMArgs m{static_cast<const uint16_t*>(q), pyr, f16, reinterpret_cast<const int32_t*>(f16 + plane), idx, score,
              p.B, p.N, p.Hq, p.Hkv, p.C, p.K, p.causal ? 1 : 0, p.scale, p.geo};
  return dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    if (std::is_same<T, uint16_t>::value) {
      const dim3 grid((unsigned)((p.N + kFlatWaves * 16 - 1) / (kFlatWaves * 16)), (unsigned)((int64_t)p.B * p.Hkv));
      PISA_LAUNCH("flat", stream, (flat_mfma_kernel<D, G>), grid, dim3(kFlatWaves * kWave), 0, m);
    } else {
      PISA_LAUNCH("flat", stream, (flat_kernel<T, D, G>), dim3((unsigned)blocks), dim3(kFlatWaves * kWave), 0, a);
    }
    return hipGetLastError();
  });
}

}  // namespace pisa
