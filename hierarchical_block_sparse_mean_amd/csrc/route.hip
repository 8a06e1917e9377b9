// Prefill routing kernels: the fused one-stage selector, stage 1 of the
// two-stage selector, and query-major block-sparse attention.
// Method: "Block Sparse Attention with Log-Linear Complexity" (PISA), hyper.ai
// page, sections "coarse-to-fine top-K selection", "kernel implementation"
// and "block-sparse attention".
#include "attend.h"
#include "kernels.h"
#include "route.h"

namespace pisa {

constexpr int kRouteWaves = 4;

struct RouteArgs {
  const void* q;
  const void* k;
  const float* pyr;
  int32_t* idx;
  float* score;
  int32_t B, N, Hq, Hkv, C, K, L;
  int32_t causal;
  int64_t cap;
  float scale;
  PyrGeom geo;
};

// Workgroup -> (b, h, first query).  Consecutive workgroups go to consecutive
// XCDs; h = bid % Hkv keeps one KV head's pyramid in one XCD's L2 when
// Hkv is a multiple of the XCD count.
__device__ __forceinline__ void map_query_block(int32_t Hkv, int32_t B, int& b, int& h, int64_t& t0) {
  const int64_t bid = blockIdx.x;
  h = (int)(bid % Hkv);
  const int64_t r = bid / Hkv;
  b = (int)(r % B);
  t0 = (r / B) * kRouteWaves;
}

template <typename T, int D, int G>
__device__ __forceinline__ void load_group_queries(const T* q, int32_t Hq, int32_t N, int b, int h, int64_t t,
                                                   float* s_q) {
  const int lane = lane_id();
  for (int i = lane; i < G * D / 8; i += kWave) {
    const int g = i / (D / 8);
    const int d = (i % (D / 8)) * 8;
    float v[8];
    load8<T>(q + (((int64_t)b * Hq + h * G + g) * N + t) * D + d, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s_q[g * D + d + e] = v[e];
  }
}

template <typename T, int D, int G, bool FUSED>
__global__ __launch_bounds__(kRouteWaves* kWave) void route_kernel(RouteArgs a) {
  __shared__ float s_q[kRouteWaves][G * D];
  __shared__ RouteLds s_r[kRouteWaves];
  const int w = threadIdx.x / kWave;
  int b, h;
  int64_t t0;
  map_query_block(a.Hkv, a.B, b, h, t0);
  const int64_t t = t0 + w;
  if (t >= a.N) return;  // wave-uniform; the kernel has no workgroup barrier
  load_group_queries<T, D, G>(static_cast<const T*>(a.q), a.Hq, a.N, b, h, t, s_q[w]);
  wave_sync();
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const T* kbase = static_cast<const T*>(a.k) + bh * a.cap * D;
  const float* pbase = a.pyr + bh * a.geo.rows * D;
  int32_t out_idx;
  float out_score;
  route_query<T, D, G>(s_r[w], s_q[w], kbase, pbase, a.geo, a.N, t, a.causal != 0, a.C, a.K, a.L, FUSED ? 1 : 2,
                       a.scale, nullptr, -1, out_idx, out_score);
  const int lane = lane_id();
  if (lane < a.K) {
    const int64_t o = (bh * a.N + t) * a.K + lane;
    a.idx[o] = out_idx;
    if (FUSED && a.score != nullptr) a.score[o] = out_score;
  }
}

hipError_t launch_route(const Problem& p, const void* q, const void* k, const float* pyr, int32_t* idx,
                        float* score, bool fused, hipStream_t stream) {
  RouteArgs a{q, k, pyr, idx, score, p.B, p.N, p.Hq, p.Hkv, p.C, p.K, p.L, p.causal ? 1 : 0, p.cap, p.scale, p.geo};
  const int64_t blocks = (int64_t)p.B * p.Hkv * ((p.N + kRouteWaves - 1) / kRouteWaves);
  return dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    if (fused)
      PISA_LAUNCH("route_fused", stream, (route_kernel<T, D, G, true>), dim3((unsigned)blocks),
                  dim3(kRouteWaves * kWave), 0, a);
    else
      PISA_LAUNCH("route_stage1", stream, (route_kernel<T, D, G, false>), dim3((unsigned)blocks),
                  dim3(kRouteWaves * kWave), 0, a);
    return hipGetLastError();
  });
}

// ---- query-major attention: one wave per (b, h, t) ------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  void* o;
  float* lse;
  int32_t B, N, Hq, Hkv, C, K;
  int32_t causal;
  int64_t cap;
  float scale;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kRouteWaves* kWave) void attn_query_kernel(AttnArgs a) {
  __shared__ float s_q[kRouteWaves][G * D];
  __shared__ AttendLds<D, G> s_a[kRouteWaves];
  const int w = threadIdx.x / kWave;
  int b, h;
  int64_t t0;
  map_query_block(a.Hkv, a.B, b, h, t0);
  const int64_t t = t0 + w;
  if (t >= a.N) return;
  load_group_queries<T, D, G>(static_cast<const T*>(a.q), a.Hq, a.N, b, h, t, s_q[w]);
  const int lane = lane_id();
  const int64_t bh = (int64_t)b * a.Hkv + h;
  if (lane < a.K) s_a[w].sel[lane] = a.idx[(bh * a.N + t) * a.K + lane];
  wave_sync();
  const T* kbase = static_cast<const T*>(a.k) + bh * a.cap * D;
  const T* vbase = static_cast<const T*>(a.v) + bh * a.cap * D;
  T* out = static_cast<T*>(a.o) + (((int64_t)b * a.Hq + h * G) * a.N + t) * D;
  float* lse = a.lse ? a.lse + ((int64_t)b * a.Hq + h * G) * a.N + t : nullptr;
  attend_query<T, D, G>(s_a[w], a.K, s_q[w], kbase, vbase, a.N, t, a.causal != 0, a.C, a.scale, nullptr, nullptr,
                        -1, out, (int64_t)a.N * D, lse, a.N);
}

hipError_t launch_attn_query(const Problem& p, const void* q, const void* k, const void* v, const int32_t* idx,
                             void* o, float* lse, hipStream_t stream) {
  AttnArgs a{q, k, v, idx, o, lse, p.B, p.N, p.Hq, p.Hkv, p.C, p.K, p.causal ? 1 : 0, p.cap, p.scale};
  const int64_t blocks = (int64_t)p.B * p.Hkv * ((p.N + kRouteWaves - 1) / kRouteWaves);
  return dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    PISA_LAUNCH("attn_query", stream, (attn_query_kernel<T, D, G>), dim3((unsigned)blocks),
                dim3(kRouteWaves * kWave), 0, a);
    return hipGetLastError();
  });
}

}  // namespace pisa
