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
// One wave per 16 / G_Q consecutive queries of one KV head: every valid leaf
// summary is scored by (16 leaves) x d x (16 query-head columns) fp16 MFMA
// tiles from the pyramid's block-floating-point copy (as in stage 1), the
// group sum is a shuffle over the G_Q columns of a query, and each query keeps
// its top K in an LDS buffer: a score enters only if it beats the current
// K-th key, and the buffer is compacted (wave sort, keep K) when it fills.
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

template <int D, int G>
__global__ __launch_bounds__(kFlatWaves* kWave) void flat_mfma_kernel(FlatMArgs a) {
  constexpr int NS = D / 32;
  constexpr int TQ = 16 / G;
  constexpr int CAP = kWave;  // candidate buffer per query
  __shared__ uint64_t s_buf[kFlatWaves][TQ][CAP];
  __shared__ int32_t s_cnt[kFlatWaves][TQ];
  __shared__ uint64_t s_thr[kFlatWaves][TQ];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const int qi = col / G, hh = col % G;
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % a.Hkv);
  const int64_t r = bid / a.Hkv;
  const int b = (int)(r % a.B);
  const int64_t t0 = ((r / a.B) * kFlatWaves + w) * TQ;
  if (t0 >= a.N) return;  // wave-uniform
  const int64_t tq = t0 + qi;
  const bool qlive = tq < a.N;
  // B operand: this column's query head, scaled into fp16 by 2^-eq
  float qv[NS][8];
  float mx = 0.f;
  if (qlive) {
    const uint16_t* qrow = a.q + (((int64_t)b * a.Hq + h * G + hh) * a.N + tq) * D;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      load8<uint16_t>(qrow + g * (D / 4) + 8 * st, qv[st]);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qv[st][e]));
    }
  } else {
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[st][e] = 0.f;
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const int eq = row_exponent(mx);
  halfx8 fq[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) fq[st][e] = to_f16_scaled(qv[st][e], eq);
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const _Float16* hb = a.f16 + (bh * a.geo.rows + a.geo.level_off[1]) * D;
  const int32_t* xb = a.ex + bh * a.geo.rows + a.geo.level_off[1];
  const int32_t M1 = (int32_t)level_rows(a.N, a.C, 1);
  // leaves valid for the last query of the tile (the others mask theirs)
  const int64_t tlast = (t0 + TQ - 1 < a.N) ? t0 + TQ - 1 : a.N - 1;
  const int32_t nl = a.causal ? (int32_t)((tlast / a.C + 1) < M1 ? (tlast / a.C + 1) : M1) : M1;
  const int32_t lq = qlive ? (a.causal ? (int32_t)((tq / a.C + 1) < M1 ? (tq / a.C + 1) : M1) : M1) : 0;
  if (lane < TQ) {
    s_cnt[w][lane] = 0;
    s_thr[w][lane] = 0ull;
  }
  wave_sync();
  for (int32_t base = 0; base < nl; base += 16) {
    const int32_t row = base + col;
    const bool vrow = row < nl;
    const int32_t er = vrow ? xb[row] : 0;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      halfx8 fa;
      if (vrow) fa = *reinterpret_cast<const halfx8*>(hb + (int64_t)row * D + g * (D / 4) + 8 * st);
      else fa = halfx8{0, 0, 0, 0, 0, 0, 0, 0};
      acc = mma16x16x32(fa, fq[st], acc);
    }
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t leaf = base + 4 * g + i;
      const int32_t eri = __shfl(er, 4 * g + i);
      float u = ldexpf(acc[i], eri + eq) * a.scale;
#pragma unroll
      for (int o = 1; o < G; o <<= 1) u += __shfl_xor(u, o);
      key[i] = (leaf < lq) ? score_key(u, leaf) : 0ull;
    }
    // append the candidates that beat the query's current K-th key
    if (hh == 0) {
      const uint64_t thr = s_thr[w][qi];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key[i] > thr) {
          const int pos = atomicAdd(&s_cnt[w][qi], 1);
          s_buf[w][qi][pos] = key[i];
        }
    }
    wave_sync();
    // compact a buffer that could overflow on the next tile
#pragma unroll
    for (int qq = 0; qq < TQ; ++qq) {
      const int cnt = s_cnt[w][qq];
      if (cnt > CAP - 16) {
        uint64_t k2 = lane < cnt ? s_buf[w][qq][lane] : 0ull;
        k2 = wave_sort_desc(k2);
        // the K-th largest key becomes the entry threshold
        const uint64_t thr = (uint64_t)(uint32_t)__shfl((int)(uint32_t)k2, a.K - 1) |
                             ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(k2 >> 32), a.K - 1) << 32);
        wave_sync();
        s_buf[w][qq][lane] = lane < a.K ? k2 : 0ull;
        if (lane == 0) {
          s_cnt[w][qq] = a.K;
          s_thr[w][qq] = thr;
        }
        wave_sync();
      }
    }
  }
  // final top K of each query, written in ascending leaf order
#pragma unroll
  for (int qq = 0; qq < TQ; ++qq) {
    const int64_t tt = t0 + qq;
    if (tt >= a.N) break;
    const int cnt = s_cnt[w][qq];
    uint64_t k2 = lane < cnt ? s_buf[w][qq][lane] : 0ull;
    k2 = wave_sort_desc(k2);
    const bool kept = lane < a.K && k2 != 0ull;
    uint64_t k3 = kept ? index_key(key_index(k2), key_score(k2)) : 0ull;
    k3 = wave_sort_desc(k3);
    if (lane < a.K) {
      const bool v = k3 != 0ull;
      const int32_t leaf = v ? index_key_index(k3) : -1;
      const int64_t o = (bh * a.N + tt) * a.K + lane;
      a.idx[o] = leaf;
      if (a.score) {
        // report the kept leaves' scores exactly: fp32 summaries x bf16 q
        float u = -INFINITY;
        if (v) {
          const float* prow = a.pyr + (bh * a.geo.rows + a.geo.level_off[1] + leaf) * D;
          u = 0.f;
#pragma unroll 1
          for (int gg = 0; gg < G; ++gg) {
            const uint16_t* qrow = a.q + (((int64_t)b * a.Hq + h * G + gg) * a.N + tt) * D;
            float acc_d = 0.f;
            for (int d = 0; d < D; d += 8) {
              float qx[8], px[8];
              load8<uint16_t>(qrow + d, qx);
              load8<float>(prow + d, px);
#pragma unroll
              for (int e = 0; e < 8; ++e) acc_d = fmaf(qx[e], px[e], acc_d);
            }
            u += acc_d * a.scale;
          }
        }
        a.score[o] = u;
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
      const int64_t tiles = (p.N + 16 / G - 1) / (16 / G);
      const int64_t mblocks = (int64_t)p.B * p.Hkv * ((tiles + kFlatWaves - 1) / kFlatWaves);
      PISA_LAUNCH("flat", stream, (flat_mfma_kernel<D, G>), dim3((unsigned)mblocks), dim3(kFlatWaves * kWave), 0,
                  m);
    } else {
      PISA_LAUNCH("flat", stream, (flat_kernel<T, D, G>), dim3((unsigned)blocks), dim3(kFlatWaves * kWave), 0, a);
    }
    return hipGetLastError();
  });
}

}  // namespace pisa
