// Wave-level coarse-to-fine routing (one wave64 per (query, KV head)).
//
// Method: "Block Sparse Attention with Log-Linear Complexity" (PISA), hyper.ai
// page.  Section "coarse-to-fine top-K selection": the descent starts from the
// single block of the coarsest level, scores at most gK candidates per level
// with the log-sum-exp block score (children = lower-level summaries, raw keys
// at the leaf level), keeps K, expands the kept blocks into their children,
// and keeps every candidate unscored when at most K are valid.  Section
// "kernel implementation": the score of a KV head is the sum of its G_Q query
// heads' scores, candidate indices stay private to the program, and the
// decode kernel walks every level down to the leaves in one program.
#pragma once

#include "common.h"

namespace pisa {

// Per-wave LDS scratch used by route_query.
struct __align__(16) RouteLds {
  int32_t cand[kWave];  // candidate block indices of the current level
  float score[kWave];   // their GQA-summed scores
  float2 fb[64];        // (scale, bias) of the rows of up to 4 tiles
};

// G dot products of one fp32 pyramid row with the G query vectors in LDS.
template <int D, int G>
__device__ __forceinline__ void dots_summary(const float* __restrict__ row, const float* s_q, float* acc) {
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll 4
  for (int d = 0; d < D; d += 8) {
    float r[8];
    load8<float>(row + d, r);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float4 qa = *reinterpret_cast<const float4*>(s_q + g * D + d);
      const float4 qb = *reinterpret_cast<const float4*>(s_q + g * D + d + 4);
      acc[g] = fmaf(r[0], qa.x, acc[g]);
      acc[g] = fmaf(r[1], qa.y, acc[g]);
      acc[g] = fmaf(r[2], qa.z, acc[g]);
      acc[g] = fmaf(r[3], qa.w, acc[g]);
      acc[g] = fmaf(r[4], qb.x, acc[g]);
      acc[g] = fmaf(r[5], qb.y, acc[g]);
      acc[g] = fmaf(r[6], qb.z, acc[g]);
      acc[g] = fmaf(r[7], qb.w, acc[g]);
    }
  }
}

// G dot products of one raw key row (dtype T) with the G query vectors in LDS.
template <typename T, int D, int G>
__device__ __forceinline__ void dots_key(const T* __restrict__ row, const float* s_q, float* acc) {
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll 4
  for (int d = 0; d < D; d += 8) {
    float r[8];
    load8<T>(row + d, r);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float4 qa = *reinterpret_cast<const float4*>(s_q + g * D + d);
      const float4 qb = *reinterpret_cast<const float4*>(s_q + g * D + d + 4);
      acc[g] = fmaf(r[0], qa.x, acc[g]);
      acc[g] = fmaf(r[1], qa.y, acc[g]);
      acc[g] = fmaf(r[2], qa.z, acc[g]);
      acc[g] = fmaf(r[3], qa.w, acc[g]);
      acc[g] = fmaf(r[4], qb.x, acc[g]);
      acc[g] = fmaf(r[5], qb.y, acc[g]);
      acc[g] = fmaf(r[6], qb.z, acc[g]);
      acc[g] = fmaf(r[7], qb.w, acc[g]);
    }
  }
}

// Score the nA candidates (LDS) of level l >= 2: u_i = sum_g LSE over the
// valid children r in {2c, 2c+1} of q_g . P_{l-1}[r] * scale.
template <int D, int G>
__device__ __forceinline__ void score_level(RouteLds& s, int nA, const float* s_q, const float* pbase,
                                            const PyrGeom& geo, int64_t n, int64_t t, bool causal, int32_t C,
                                            int32_t l, float scale) {
  const int lane = lane_id();
  const int64_t m_child = level_rows(n, C, l - 1);
  const int64_t child_span = (int64_t)C << (l - 2);
  const float* child_level = pbase + geo.level_off[l - 1] * D;
  for (int base = 0; base < 2 * nA; base += kWave) {
    const int c = base + lane;
    const int i = c >> 1;
    const int64_t r = (i < nA) ? 2 * (int64_t)s.cand[i] + (c & 1) : -1;
    const bool valid = (i < nA) && r < m_child && (!causal || r * child_span <= t);
    float logit[G];
    if (valid) {
      dots_summary<D, G>(child_level + r * D, s_q, logit);
#pragma unroll
      for (int g = 0; g < G; ++g) logit[g] *= scale;
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) logit[g] = -INFINITY;
    }
    float u = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) u += lse2(logit[g], __shfl_xor(logit[g], 1));
    if ((c & 1) == 0 && i < nA) s.score[i] = u;
  }
}

// Score the nA candidate leaves (LDS) by the exact raw-key LSE summed over the
// group: one leaf at a time, lanes over its keys.
template <typename T, int D, int G>
__device__ __forceinline__ void score_leaves(RouteLds& s, int nA, const float* s_q, const T* kbase, int64_t n,
                                             int64_t t, bool causal, int32_t C, float scale,
                                             const T* extra_row, int64_t extra_pos) {
  const int lane = lane_id();
  for (int i = 0; i < nA; ++i) {
    const int64_t j = s.cand[i];
    const int64_t lo = j * C;
    int64_t hi = lo + C < n ? lo + C : n;
    if (causal && hi > t + 1) hi = t + 1;
    float m[G], e[G];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -INFINITY;
    float logit0[G], logit1[G];
    const int64_t key0 = lo + lane, key1 = lo + kWave + lane;
    const bool v0 = key0 < hi, v1 = key1 < hi;
    if (v0) {
      dots_key<T, D, G>(key0 == extra_pos ? extra_row : kbase + key0 * D, s_q, logit0);
#pragma unroll
      for (int g = 0; g < G; ++g) logit0[g] *= scale;
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) logit0[g] = -INFINITY;
    }
    if (v1) {
      dots_key<T, D, G>(key1 == extra_pos ? extra_row : kbase + key1 * D, s_q, logit1);
#pragma unroll
      for (int g = 0; g < G; ++g) logit1[g] *= scale;
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) logit1[g] = -INFINITY;
    }
    float u = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = wave_max(fmaxf(logit0[g], logit1[g]));
      e[g] = (v0 ? __expf(logit0[g] - m[g]) : 0.f) + (v1 ? __expf(logit1[g] - m[g]) : 0.f);
      e[g] = wave_sum(e[g]);
      u += m[g] + __logf(e[g]);
    }
    if (lane == 0) s.score[i] = u;
  }
}

// The descent for one query.  Levels L .. l_stop (l_stop = 1: fused, leaf
// level scored on raw keys; l_stop = 2: stage 1, ends with the kept level-2
// blocks).  On return lane i < K holds the i-th kept block (ascending index)
// and its score, or -1 / -inf.
//   n: tokens that define level sizes; t: query position; causal: validity
//   rule (decode passes t = n - 1 with causal set, where every block is valid).
//   extra_row / extra_pos: a key row to use instead of kbase row extra_pos
//   (decode's new token), or extra_pos = -1.
template <typename T, int D, int G>
__device__ void route_query(RouteLds& s, const float* s_q, const T* kbase, const float* pbase, const PyrGeom& geo,
                            int64_t n, int64_t t, bool causal, int32_t C, int32_t K, int32_t L, int32_t l_stop,
                            float scale, const T* extra_row, int64_t extra_pos, int32_t& out_idx,
                            float& out_score) {
  const int lane = lane_id();
  int nA = 1;
  if (lane == 0) s.cand[0] = 0;
  int32_t kept = (lane == 0) ? 0 : -1;
  float kept_score = -INFINITY;
  int nI = 1;
  wave_sync();
  for (int32_t l = L; l >= l_stop; --l) {
    const int64_t ml = level_rows(n, C, l);
    const int64_t span = (int64_t)C << (l - 1);
    // drop invalid candidates, compacting the list
    const int32_t j = (lane < nA) ? s.cand[lane] : -1;
    const bool valid = j >= 0 && j < ml && (!causal || (int64_t)j * span <= t);
    const uint64_t mask = __ballot(valid);
    const int pos = __popcll(mask & ((1ull << lane) - 1ull));
    nA = __popcll(mask);
    wave_sync();
    if (valid) s.cand[pos] = j;
    wave_sync();
    if (nA > K || l == 1) {
      if (l >= 2)
        score_level<D, G>(s, nA, s_q, pbase, geo, n, t, causal, C, l, scale);
      else
        score_leaves<T, D, G>(s, nA, s_q, kbase, n, t, causal, C, scale, extra_row, extra_pos);
      wave_sync();
      uint64_t key = (lane < nA) ? score_key(s.score[lane], s.cand[lane]) : 0ull;
      key = wave_sort_desc(key);
      nI = nA < K ? nA : K;
      kept = (lane < nI) ? key_index(key) : -1;
      kept_score = (lane < nI) ? key_score(key) : -INFINITY;
    } else {
      nI = nA;
      kept = (lane < nA) ? s.cand[lane] : -1;
    }
    if (l > l_stop) {
      wave_sync();
      if (lane < nI) {
        s.cand[2 * lane] = 2 * kept;
        s.cand[2 * lane + 1] = 2 * kept + 1;
      }
      nA = 2 * nI;
      wave_sync();
    }
  }
  uint64_t k2 = (lane < nI) ? index_key(kept, kept_score) : 0ull;
  k2 = wave_sort_desc(k2);
  out_idx = (lane < nI) ? index_key_index(k2) : -1;
  out_score = (lane < nI) ? index_key_score(k2) : -INFINITY;
}

}  // namespace pisa
