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

hipError_t launch_flat(const Problem& p, const void* q, const float* pyr, int32_t* idx, float* score,
                       hipStream_t stream) {
  FlatArgs a{q, pyr, idx, score, p.B, p.N, p.Hq, p.Hkv, p.C, p.K, p.causal ? 1 : 0, p.scale, p.geo};
  const int64_t blocks = (int64_t)p.B * p.Hkv * ((p.N + kFlatWaves - 1) / kFlatWaves);
  return dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    PISA_LAUNCH("flat", stream, (flat_kernel<T, D, G>), dim3((unsigned)blocks), dim3(kFlatWaves * kWave), 0, a);
    return hipGetLastError();
  });
}

}  // namespace pisa
