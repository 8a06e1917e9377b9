// Wave-level block-sparse softmax attention for one (query, KV head): the
// G_Q query heads of the group attend over the raw keys/values of the kept
// leaves ("Block Sparse Attention with Log-Linear Complexity", hyper.ai page,
// section "block-sparse attention", the o_t equation), with an online softmax.
#pragma once

#include "common.h"
#include "route.h"

namespace pisa {

template <int D, int G>
struct AttendLds {
  float p[G][kWave];  // probabilities of the current 64-key chunk
  int32_t sel[kWave]; // kept leaves
};

// Output dims owned by a lane: DPL consecutive dims starting at lane * DPL.
template <typename T, int DPL>
__device__ __forceinline__ void load_dims(const T* p, float* out);
template <>
__device__ __forceinline__ void load_dims<uint16_t, 2>(const uint16_t* p, float* out) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  out[0] = __uint_as_float(w << 16);
  out[1] = __uint_as_float(w & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load_dims<uint16_t, 1>(const uint16_t* p, float* out) { out[0] = bf16_to_f32(*p); }
template <>
__device__ __forceinline__ void load_dims<float, 2>(const float* p, float* out) {
  const float2 w = *reinterpret_cast<const float2*>(p);
  out[0] = w.x;
  out[1] = w.y;
}
template <>
__device__ __forceinline__ void load_dims<float, 1>(const float* p, float* out) { out[0] = *p; }

// s_q: [G][D] fp32 queries in LDS; a.sel[0..nsel) kept leaves (-1 entries
// skipped).  Keys i of leaf j: [jC, min(jC + C, n)), and i <= t when causal.
// extra_k/extra_v replace the rows at position extra_pos (or extra_pos = -1).
// Writes out[g * out_stride + d] and, if lse_out, lse_out[g * lse_stride].
template <typename T, int D, int G>
__device__ void attend_query(AttendLds<D, G>& a, int nsel, const float* s_q, const T* kbase, const T* vbase,
                             int64_t n, int64_t t, bool causal, int32_t C, float scale, const T* extra_k,
                             const T* extra_v, int64_t extra_pos, T* out, int64_t out_stride, float* lse_out,
                             int64_t lse_stride) {
  constexpr int DPL = D / kWave;
  const int lane = lane_id();
  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[g][e] = 0.f;
  }
  for (int s = 0; s < nsel; ++s) {
    const int64_t j = a.sel[s];
    if (j < 0) continue;
    const int64_t lo = j * C;
    int64_t hi = lo + C < n ? lo + C : n;
    if (causal && hi > t + 1) hi = t + 1;
    for (int64_t base = lo; base < hi; base += kWave) {
      const int64_t key = base + lane;
      const bool valid = key < hi;
      float logit[G];
      if (valid) {
        dots_key<T, D, G>(key == extra_pos ? extra_k : kbase + key * D, s_q, logit);
#pragma unroll
        for (int g = 0; g < G; ++g) logit[g] *= scale;
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) logit[g] = -INFINITY;
      }
      float alpha[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], wave_max(logit[g]));
        alpha[g] = (m[g] == -INFINITY) ? 0.f : __expf(m[g] - mn);
        const float pv = valid ? __expf(logit[g] - mn) : 0.f;
        l[g] = l[g] * alpha[g] + wave_sum(pv);
        m[g] = mn;
        a.p[g][lane] = pv;
      }
      wave_sync();
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[g][e] *= alpha[g];
      const int cnt = (int)((hi - base) < kWave ? (hi - base) : kWave);
      for (int kk = 0; kk < cnt; ++kk) {
        const int64_t key_i = base + kk;
        const T* vrow = (key_i == extra_pos) ? extra_v : vbase + key_i * D;
        float vv[DPL];
        load_dims<T, DPL>(vrow + lane * DPL, vv);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pg = a.p[g][kk];
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[g][e] = fmaf(pg, vv[e], o[g][e]);
        }
      }
      wave_sync();
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float inv = (l[g] > 0.f) ? 1.f / l[g] : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) store1<T>(out + g * out_stride + lane * DPL + e, o[g][e] * inv);
    if (lse_out != nullptr && lane == 0)
      lse_out[g * lse_stride] = (l[g] > 0.f) ? m[g] + __logf(l[g]) : -INFINITY;
  }
}

}  // namespace pisa
