// Fused decode step ("Block Sparse Attention with Log-Linear Complexity",
// hyper.ai page, section "kernel implementation", decode paragraph: the mean
// pyramid is cached, each new token updates only the current leaf mean and
// its ancestor path, and one fused program walks from the coarsest level down
// to the leaves, scoring raw key blocks directly).  Attention over the kept
// leaves runs in the same program.
//
// One wave per (sequence, KV head).  The new token's k/v rows are appended to
// the caches; the current leaf's mean is recomputed from its raw keys (so the
// cached pyramid stays equal to a rebuild over the prefix), then each
// ancestor on the path is recomputed from its children.
#include "attend.h"
#include "kernels.h"
#include "route.h"

namespace pisa {

struct DecodeKArgs {
  void* k_cache;
  void* v_cache;
  float* pyr;
  _Float16* f16;  // block-floating-point copy of the summaries
  int32_t* ex;    // its per-row exponents
  const int32_t* len;
  const void* q_new;
  const void* k_new;
  const void* v_new;
  void* o;
  int32_t* idx;
  float* score;
  int32_t* err;
  int32_t S, Hq, Hkv, C, K;
  int64_t cap;
  float scale;
  PyrGeom geo;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kWave) void decode_kernel(DecodeKArgs a) {
  __shared__ float s_q[G * D];
  __shared__ RouteLds s_r;
  __shared__ AttendLds<D, G> s_a;
  constexpr int DPL = D / kWave;
  const int lane = lane_id();
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % a.Hkv);
  const int s = (int)(bid / a.Hkv);
  const int64_t n = a.len[s];
  if (n < 0 || n >= a.cap) {
    if (lane == 0 && a.err != nullptr) a.err[0] = 1;
    return;
  }
  const int64_t n1 = n + 1;
  const int64_t sh = (int64_t)s * a.Hkv + h;
  T* kbase = static_cast<T*>(a.k_cache) + sh * a.cap * D;
  T* vbase = static_cast<T*>(a.v_cache) + sh * a.cap * D;
  const T* knew = static_cast<const T*>(a.k_new) + sh * D;
  const T* vnew = static_cast<const T*>(a.v_new) + sh * D;
  float* pbase = a.pyr + sh * a.geo.rows * D;
  _Float16* hbase = a.f16 + sh * a.geo.rows * D;
  int32_t* xbase = a.ex + sh * a.geo.rows;
  // writes summary row `row` (this lane's DPL dims in v) and its fp16 copy
  auto put_row = [&](int64_t row, const float* v) {
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      pbase[row * D + lane * DPL + e] = v[e];
      mx = fmaxf(mx, fabsf(v[e]));
    }
    const int ex = row_exponent(wave_max(mx));
#pragma unroll
    for (int e = 0; e < DPL; ++e) hbase[row * D + lane * DPL + e] = to_f16_scaled(v[e], ex);
    if (lane == 0) xbase[row] = ex;
  };

  // 1. append k, v at row n
  for (int d = lane; d < D; d += kWave) {
    kbase[n * D + d] = knew[d];
    vbase[n * D + d] = vnew[d];
  }
  // 2. leaf mean of leaf n / C over its raw keys (the new key read from k_new)
  const int64_t j = n / a.C;
  const int64_t lo = j * a.C;
  const float cnt = (float)(n1 - lo);
  float cur[DPL];
  {
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    for (int64_t i = lo; i < n; ++i) {
      float v[DPL];
      load_dims<T, DPL>(kbase + i * D + lane * DPL, v);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += v[e];
    }
    float v[DPL];
    load_dims<T, DPL>(knew + lane * DPL, v);
#pragma unroll
    for (int e = 0; e < DPL; ++e) cur[e] = (acc[e] + v[e]) / cnt;
    put_row(a.geo.level_off[1] + j, cur);
  }
  // 3. ancestors: node j >> (l-1) of level l is the mean of its existing children
  const int32_t L1 = num_levels(n1, a.C);
  int64_t node = j;
  for (int32_t l = 2; l <= L1; ++l) {
    const int64_t sib = node ^ 1;
    const int64_t m_child = level_rows(n1, a.C, l - 1);
    const float* child_level = pbase + a.geo.level_off[l - 1] * D;
    if (sib < m_child) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float o = child_level[sib * D + lane * DPL + e];
        cur[e] = (node & 1) ? (o + cur[e]) * 0.5f : (cur[e] + o) * 0.5f;
      }
    }
    node >>= 1;
    put_row(a.geo.level_off[l] + node, cur);
  }
  __threadfence();  // the path rows are read back below by this wave

  // 4. fused selection for the new query at t = n (every block is valid)
  const T* qn = static_cast<const T*>(a.q_new) + ((int64_t)s * a.Hq + h * G) * D;
  for (int i = lane; i < G * D; i += kWave) s_q[i] = load1<T>(qn + i);
  wave_sync();
  int32_t out_idx;
  float out_score;
  route_query<T, D, G>(s_r, s_q, kbase, pbase, a.geo, n1, n, true, a.C, a.K, L1, 1, a.scale, knew, n, out_idx,
                       out_score);
  if (lane < a.K) {
    if (a.idx) a.idx[sh * a.K + lane] = out_idx;
    if (a.score) a.score[sh * a.K + lane] = out_score;
    s_a.sel[lane] = out_idx;
  }
  wave_sync();
  // 5. attention of the G query heads over the kept leaves
  T* out = static_cast<T*>(a.o) + ((int64_t)s * a.Hq + h * G) * D;
  attend_query<T, D, G>(s_a, a.K, s_q, kbase, vbase, n1, n, true, a.C, a.scale, knew, vnew, n, out, D, nullptr, 0);
}

__global__ void decode_bump_kernel(int32_t* len, int32_t S, int64_t cap) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S && len[s] >= 0 && len[s] < cap) len[s] += 1;
}

hipError_t launch_decode(const DecodeArgs& d, void* k_cache, void* v_cache, float* pyr, int32_t* len,
                         const void* q_new, const void* k_new, const void* v_new, void* o, int32_t* idx,
                         float* score, int32_t* err, hipStream_t stream) {
  const int64_t plane = (int64_t)d.S * d.Hkv * d.geo.rows * d.D;
  _Float16* f16 = reinterpret_cast<_Float16*>(pyr + plane);
  DecodeKArgs a{k_cache, v_cache, pyr, f16, reinterpret_cast<int32_t*>(f16 + plane), len, q_new, k_new, v_new, o, idx, score, err,
                d.S, d.Hq, d.Hkv, d.C, d.K, d.cap, d.scale, d.geo};
  hipError_t e = dispatch_tdg(d.dtype, d.D, d.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    PISA_LAUNCH("decode", stream, (decode_kernel<T, D, G>), dim3((unsigned)((int64_t)d.S * d.Hkv)), dim3(kWave), 0,
                a);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  PISA_LAUNCH("decode_bump", stream, decode_bump_kernel, dim3((d.S + 255) / 256), dim3(256), 0, len, d.S, d.cap);
  return hipGetLastError();
}

}  // namespace pisa
