// Fused decode step ("Block Sparse Attention with Log-Linear Complexity",
// hyper.ai page, section "kernel implementation", decode paragraph: the mean
// pyramid is cached, each new token updates only the current leaf mean and
// its ancestor path, and one fused program walks from the coarsest level down
// to the leaves, scoring raw key blocks directly).  Attention over the kept
// leaves runs in the same program.
//
// One workgroup of NW waves per (sequence, KV head):
//   1. append k, v at row n; the current leaf's mean from its raw keys (rows
//      summed across the waves), then each ancestor on the path from its
//      children (sibling rows fetched by all waves at once), so the cached
//      pyramid stays equal to a rebuild over the prefix;
//   2. the descent for the new query (t = n, every block valid): the child
//      rows of a scored level are spread over all waves, 8 lanes per row of
//      the pyramid's fp16 block-floating-point copy (row * 2^-ex, half the
//      bytes of the fp32 row; the same rows prefill stage 1 scores); wave 0
//      keeps the top K and expands them;
//   3. leaf level: each candidate leaf's C raw keys against the G_Q query
//      heads on MFMA (keys as rows, heads as columns), its per-head max and
//      log-sum-exp kept in LDS, and, where they fit, its raw logits too;
//      wave 0 keeps the final top K;
//   4. attention: the per-head max and denominator over the kept leaves come
//      from those LDS values, so every wave's partial output over its leaves
//      is already on the common scale; partials add through LDS.  The kept
//      leaves' logits are read back from LDS (their keys are not fetched a
//      second time), so only their values are read here.
#include "kernels.h"

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

constexpr int kDecMaxCand = 64;  // 2K, K <= 32
// raw logits of the candidate leaves kept in LDS for the attention phase
// (2K candidates x C keys x G_Q heads; 32 KB: K = 16, C = 64, G_Q = 4);
// larger problems recompute the kept leaves' logits from their keys
constexpr int kDecLogitFloats = 8192;
// value rows per lane whose loads are in flight together in the attention
// phase (8 would spill at d = 128, G_Q = 4)
constexpr int kVRows = 4;

// N consecutive elements (N = 4 or 8) as fp32
template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* p, float* out) {
  if constexpr (N == 8) {
    load8<T>(p, out);
  } else if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(u.x << 16);
    out[1] = __uint_as_float(u.x & 0xFFFF0000u);
    out[2] = __uint_as_float(u.y << 16);
    out[3] = __uint_as_float(u.y & 0xFFFF0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(p);
    out[0] = f.x;
    out[1] = f.y;
    out[2] = f.z;
    out[3] = f.w;
  }
}

// Raw dot products of the keys [lo, hi) of one leaf with the G query heads:
// S^T tile kb holds keys lo + 16kb + 4(lane/16) + i (i = 0..3) in column
// lane % 16 = head.  Row newpos is read from knew (the appended token).
template <typename T, int D, int NKB>
__device__ __forceinline__ void leaf_dots(const Frag<T>* fq, const T* kbase, const T* knew, int64_t newpos, int64_t lo,
                                          int64_t hi, floatx4* acc) {
  constexpr int NS = D / 32;
  const int lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const int nk = (int)(hi - lo), knew_off = (int)(newpos - lo);  // keys of the leaf; the new key's offset
  const T* leaf = kbase + lo * D;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int r = kb * 16 + col;
    const T* row = (r == knew_off) ? knew : leaf + r * D;
    Frag<T> fk[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (r < nk) fk[s].load_nt(row + 32 * s + 8 * g);  // contiguous 64-byte spans per row (streamed)
      else fk[s].zero();
    }
    acc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[kb] = mma(fk[s], fq[s], acc[kb]);
    // at most two key blocks of fragments in flight (register budget)
    if (kb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, int D, int G, int NW, int NKB>
// two workgroups per CU where the registers allow it (bf16, C <= 64)
__global__ __launch_bounds__(NW* kWave, (sizeof(T) == 2 && NKB <= 4) ? NW / 2 : NW / 4) void decode_kernel(DecodeKArgs a) {
  constexpr int DPL = D / kWave;  // dims per lane in whole-row work
  constexpr int NS = D / 32;
  constexpr int CP = NKB * 16;    // keys per leaf tile
  constexpr int DPV = G >= 8 ? 4 : 8;  // dims per lane in the PV product
  constexpr int LPR = D / DPV;         // lanes per V row there
  constexpr int RPI = kWave / LPR;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __align__(16) float s_q[G * D];
  __shared__ int32_t s_cand[kDecMaxCand];
  __shared__ float s_score[kDecMaxCand];
  __shared__ float s_lm[kDecMaxCand][G];  // per candidate leaf and head: max logit
  __shared__ float s_ll[kDecMaxCand][G];  // and log-sum-exp
  __shared__ int32_t s_sel[32], s_slot[32];
  __shared__ float s_M[G], s_L[G];
  __shared__ int32_t s_state[2];  // level, candidate count
  __shared__ __align__(16) float s_p[NW][CP][G];
  __shared__ float s_logit[kDecLogitFloats];  // [candidate][key][head] raw dot products
  constexpr int kUpdFloats = NW * D + (kMaxLevels + 1) * D;  // leaf-mean partials + sibling rows
  constexpr int kOutFloats = NW * G * D;                     // partial outputs
  __shared__ __align__(16) float s_u[kUpdFloats > kOutFloats ? kUpdFloats : kOutFloats];
  float* s_mean = s_u;           // [NW][D]
  float* s_sib = s_u + NW * D;   // [level][D]
  float* s_o = s_u;              // [NW][G][D], after the update phase

  const int w = threadIdx.x / kWave, lane = lane_id();
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % a.Hkv);
  const int s = (int)(bid / a.Hkv);
  const int64_t n = a.len[s];
  if (n < 0 || n >= a.cap) {  // uniform over the workgroup
    if (threadIdx.x == 0 && a.err != nullptr) a.err[0] = 1;
    return;
  }
  const int64_t n1 = n + 1;
  const int C = a.C, K = a.K;
  const int64_t sh = (int64_t)s * a.Hkv + h;
  T* kbase = static_cast<T*>(a.k_cache) + sh * a.cap * D;
  T* vbase = static_cast<T*>(a.v_cache) + sh * a.cap * D;
  const T* knew = static_cast<const T*>(a.k_new) + sh * D;
  const T* vnew = static_cast<const T*>(a.v_new) + sh * D;
  const T* qn = static_cast<const T*>(a.q_new) + ((int64_t)s * a.Hq + h * G) * D;
  float* pbase = a.pyr + sh * a.geo.rows * D;
  _Float16* hbase = a.f16 + sh * a.geo.rows * D;
  int32_t* xbase = a.ex + sh * a.geo.rows;

  // ---- 1. append, leaf mean, ancestor path ---------------------------------
  const int64_t j_leaf = n / C;
  const int64_t lo_leaf = j_leaf * C;
  const int32_t L1 = num_levels(n1, C);
  if (w == 0)
    for (int d = lane; d < D; d += kWave) {
      kbase[n * D + d] = knew[d];
      vbase[n * D + d] = vnew[d];
    }
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) s_q[i] = load1<T>(qn + i);
  {
    // cached rows of the current leaf: 8 lanes per row, 8 rows per wave
    constexpr int DL = D / 8;
    const int sub = lane & 7;
    float acc[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[e] = 0.f;
    for (int64_t i = lo_leaf + w * 8 + (lane >> 3); i < n; i += NW * 8) {
#pragma unroll
      for (int e = 0; e < DL; e += 8) {
        float v[8];
        load8<T>(kbase + i * D + sub * DL + e, v);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[e + x] += v[x];
      }
    }
#pragma unroll
    for (int e = 0; e < DL; ++e)
#pragma unroll
      for (int o = 8; o < kWave; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
    if (lane < 8)
#pragma unroll
      for (int e = 0; e < DL; ++e) s_mean[w * D + sub * DL + e] = acc[e];
    // sibling of the path node at level l - 1, for l = 2 .. L1
    for (int32_t l = 2 + w; l <= L1; l += NW) {
      const int64_t node = j_leaf >> (l - 2);
      const int64_t sib = node ^ 1;
      if (sib < level_rows(n1, C, l - 1)) {
        const float* row = pbase + (a.geo.level_off[l - 1] + sib) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_sib[l * D + lane * DPL + e] = row[lane * DPL + e];
      }
    }
  }
  __syncthreads();
  if (w == 0) {
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
    const float cnt = (float)(n1 - lo_leaf);
    float cur[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      float acc = 0.f;
      for (int ww = 0; ww < NW; ++ww) acc += s_mean[ww * D + lane * DPL + e];
      cur[e] = (acc + load1<T>(knew + lane * DPL + e)) / cnt;
    }
    put_row(a.geo.level_off[1] + j_leaf, cur);
    int64_t node = j_leaf;
    for (int32_t l = 2; l <= L1; ++l) {
      if ((node ^ 1) < level_rows(n1, C, l - 1)) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) cur[e] = (cur[e] + s_sib[l * D + lane * DPL + e]) * 0.5f;
      }
      node >>= 1;
      put_row(a.geo.level_off[l] + node, cur);
    }
  }
  // the path rows are read below by every wave of this workgroup, which all
  // run on one CU: a workgroup-scope fence suffices (no L2 write-back)
  __threadfence_block();
  __syncthreads();

  // top K of the keys in lanes [0, 2K) into lanes [0, K) (half sorts for K = 16
  // or 32, unordered; a full wave sort otherwise), and a descending sort of
  // lanes [0, K)
  auto topk_keys = [&](uint64_t key) -> uint64_t {
    if (K == 16) return top_half<16>(key);
    if (K == 32) return top_half<32>(key);
    return wave_sort_desc(key);
  };
  auto sort_k = [&](uint64_t key) -> uint64_t {
    if (K == 16) return group_sort_desc<16>(key);
    if (K == 32) return group_sort_desc<32>(key);
    return wave_sort_desc(key);
  };

  // ---- 2. descent, levels L1 .. 2 ----------------------------------------
  // wave 0: drop candidates beyond the level's rows (every block starts at or
  // before t = n), compacting the list; returns the new count
  auto compact = [&](int nA, int64_t ml) -> int {
    const int32_t j = lane < nA ? s_cand[lane] : -1;
    const bool valid = j >= 0 && j < ml;
    const uint64_t mask = __ballot(valid);
    const int pos = __popcll(mask & ((1ull << lane) - 1ull));
    wave_sync();
    if (valid) s_cand[pos] = j;
    wave_sync();
    return __popcll(mask);
  };
  // wave 0: replace the first nI candidates (in lanes' `kept`) by their children
  auto expand = [&](int32_t kept, int nI) {
    wave_sync();
    if (lane < nI) {
      s_cand[2 * lane] = 2 * kept;
      s_cand[2 * lane + 1] = 2 * kept + 1;
    }
    wave_sync();
  };
  if (w == 0) {
    int l = L1, nA = 1;
    if (lane == 0) s_cand[0] = 0;
    wave_sync();
    // levels with at most K candidates keep them all unscored
    while (l >= 2 && nA <= K) {
      const int32_t kept = lane < nA ? s_cand[lane] : -1;
      expand(kept, nA);
      --l;
      nA = compact(2 * nA, level_rows(n1, C, l));
    }
    if (lane == 0) {
      s_state[0] = l;
      s_state[1] = nA;
    }
  }
  __syncthreads();
  // this lane's slice of the G query rows (dims sub*DL .. +DL), held in
  // registers through the descent where they fit
  constexpr int DLq = D / 8;
  constexpr bool QREG = G * DLq <= 64;
  float qr[QREG ? G : 1][QREG ? DLq : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < DLq; ++e) qr[g][e] = s_q[g * D + (lane & 7) * DLq + e];
  }
  for (;;) {
    const int l = s_state[0], nA = s_state[1];
    if (l < 2) break;
    // score the nA > K candidates of level l by their children at level l - 1
    {
      const int64_t m_child = level_rows(n1, C, l - 1);
      const _Float16* child_level = hbase + a.geo.level_off[l - 1] * D;
      const int32_t* child_ex = xbase + a.geo.level_off[l - 1];
      constexpr int DL = D / 8;  // dims per lane, 8 lanes per row
      const int sub = lane & 7;
      for (int base = 0; base < 2 * nA; base += NW * 8) {
        const int rr = base + w * 8 + (lane >> 3);
        const int i = rr >> 1;
        int32_t ci = s_cand[i & (kDecMaxCand - 1)];
        asm volatile("" : "+v"(ci));
        const int64_t r = (i < nA) ? 2 * (int64_t)ci + (rr & 1) : -1;
        const bool valid = i < nA && r < m_child;
        const int64_t rl = valid ? r : 0;  // rows past the list load row 0 (results dropped below)
        float dot[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = 0.f;
        int32_t er = child_ex[rl];
        {
          const _Float16* row = child_level + rl * D + sub * DL;
          float rv[DL];
#pragma unroll
          for (int e = 0; e < DL; e += 8) {
            const halfx8 x = *reinterpret_cast<const halfx8*>(row + e);
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) rv[e + c8] = (float)x[c8];
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < DL; e += 4) {
              float4 qv;
              if constexpr (QREG) qv = float4{qr[g][e], qr[g][e + 1], qr[g][e + 2], qr[g][e + 3]};
              else qv = *reinterpret_cast<const float4*>(s_q + g * D + sub * DL + e);
              dot[g] = fmaf(rv[e], qv.x, dot[g]);
              dot[g] = fmaf(rv[e + 1], qv.y, dot[g]);
              dot[g] = fmaf(rv[e + 2], qv.z, dot[g]);
              dot[g] = fmaf(rv[e + 3], qv.w, dot[g]);
            }
        }
        // the row is stored as row * 2^-er: its logits scale by 2^er
        const float rscale = ldexpf(a.scale, er);
        float u = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float x = valid ? group_sum<8>(dot[g]) * rscale : -INFINITY;
          u += lse2(x, __shfl_xor(x, 8));  // the sibling child sits 8 lanes away
        }
        if ((lane & 15) == 0 && i < nA) s_score[i] = u;
      }
    }
    __syncthreads();
    if (w == 0) {
      uint64_t key = (lane < nA) ? score_key(s_score[lane], s_cand[lane]) : 0ull;
      key = topk_keys(key);  // nA > K here: lanes [0, K) all hold kept blocks
      int nI = nA < K ? nA : K;
      int32_t kept = (lane < nI) ? key_index(key) : -1;
      int ll = l, na = nI;
      expand(kept, na);
      --ll;
      na = compact(2 * na, level_rows(n1, C, ll));
      while (ll >= 2 && na <= K) {
        kept = lane < na ? s_cand[lane] : -1;
        expand(kept, na);
        --ll;
        na = compact(2 * na, level_rows(n1, C, ll));
      }
      if (lane == 0) {
        s_state[0] = ll;
        s_state[1] = na;
      }
    }
    __syncthreads();
  }

  // ---- 3. leaf level: raw-key log-sum-exp per candidate leaf ----------------
  const int nA = s_state[1];
  const int g4 = lane >> 4, col = lane & 15;
  Frag<T> fq[NS];  // B operand: column col = query head col of the group
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    if (col < G) fq[st].load(qn + col * D + 32 * st + 8 * g4);  // element order of leaf_dots
    else fq[st].zero();
  }
  const float sl2 = a.scale * kLog2e;
  // the candidates' raw logits stay in LDS for the attention phase if they fit
  const bool keep_logits = nA * CP * G <= kDecLogitFloats;
  for (int i = w; i < nA; i += NW) {
    const int64_t lo = (int64_t)s_cand[i] * C;
    const int64_t hi = lo + C < n1 ? lo + C : n1;
    const int nk = (int)(hi - lo);
    floatx4 acc[NKB];
    leaf_dots<T, D, NKB>(fq, kbase, knew, n, lo, hi, acc);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = kb * 16 + 4 * g4 + e < nk;
        acc[kb][e] = ok ? acc[kb][e] : -INFINITY;
        mx = fmaxf(mx, acc[kb][e]);
      }
    if (keep_logits && col < G)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_logit[(i * CP + kb * 16 + 4 * g4 + e) * G + col] = acc[kb][e];
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += exp2_nonpos((acc[kb][e] - mx) * sl2);  // exp2(-inf) = 0
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    const float m_nat = mx * a.scale;
    const float lse = m_nat + __logf(sum);
    if (g4 == 0 && col < G) {
      s_lm[i][col] = m_nat;
      s_ll[i][col] = lse;
    }
    const float u = group_sum<16>((g4 == 0 && col < G) ? lse : 0.f);
    if (lane == 0) s_score[i] = u;
  }
  __syncthreads();
  if (w == 0) {
    uint64_t key = (lane < nA) ? score_key(s_score[lane], s_cand[lane]) : 0ull;
    key = topk_keys(key);
    const int nI = nA < K ? nA : K;
    // the kept leaves are the nonzero keys of lanes [0, K) (nA may be < K)
    const bool kv = lane < K && key != 0ull;
    const int32_t kept = kv ? key_index(key) : -1;
    const float kept_score = kv ? key_score(key) : -INFINITY;
    uint64_t k2 = kv ? index_key(kept, kept_score) : 0ull;
    k2 = sort_k(k2);
    const int32_t out_idx = (lane < nI) ? index_key_index(k2) : -1;
    const float out_score = (lane < nI) ? index_key_score(k2) : -INFINITY;
    if (lane < K) {
      if (a.idx) a.idx[sh * K + lane] = out_idx;
      if (a.score) a.score[sh * K + lane] = out_score;
    }
    if (lane < nI) {
      int slot = 0;
      for (int c = 0; c < nA; ++c)
        if (s_cand[c] == out_idx) slot = c;
      s_sel[lane] = out_idx;
      s_slot[lane] = slot;
    }
    wave_sync();
    if (lane < G) {
      float M = -INFINITY;
      for (int c = 0; c < nI; ++c) M = fmaxf(M, s_lm[s_slot[c]][lane]);
      float L = 0.f;
      for (int c = 0; c < nI; ++c) L += __expf(s_ll[s_slot[c]][lane] - M);
      s_M[lane] = M;
      s_L[lane] = L;
    }
    if (lane == 0) s_state[1] = nI;
  }
  __syncthreads();

  // ---- 4. attention over the kept leaves -----------------------------------
  const int nI = s_state[1];
  const float mcol = col < G ? s_M[col] * kLog2e : 0.f;
  const int rg = lane / LPR, dl = (lane % LPR) * DPV;
  // this wave's partial output accumulates in its own LDS slice, so the
  // accumulators are not live while the next leaf's keys are in flight
  for (int i = lane; i < G * D; i += kWave) s_o[w * G * D + i] = 0.f;
  wave_sync();
  for (int c = w; c < nI; c += NW) {
    const int64_t lo = (int64_t)s_sel[c] * C;
    const int64_t hi = lo + C < n1 ? lo + C : n1;
    const int nk = (int)(hi - lo);
    if (keep_logits) {
      // p from the logits phase 3 left in LDS (lane = key group x head, the
      // same arithmetic as from recomputed dot products)
      const int slot = s_slot[c];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb * 16 + 4 * g4 + e;
          if (col < G) {
            const float x = s_logit[(slot * CP + key) * G + col];
            s_p[w][key][col] = key < nk ? exp2_nonpos(fmaf(x, sl2, -mcol)) : 0.f;
          }
        }
    } else {
      floatx4 acc[NKB];
      leaf_dots<T, D, NKB>(fq, kbase, knew, n, lo, hi, acc);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb * 16 + 4 * g4 + e;
          const float p = key < nk ? exp2_nonpos(fmaf(acc[kb][e], sl2, -mcol)) : 0.f;
          if (col < G) s_p[w][key][col] = p;
        }
    }
    wave_sync();
    float acc_o[G][DPV];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < DPV; ++e) acc_o[g][e] = 0.f;
    // kVRows value rows per lane in flight: every load of a batch is issued
    // before the first is used (rows past the leaf re-read row rg, which
    // exists whenever the loop runs); each lane's DPV elements of a row are
    // read as 16- or 8-byte pieces
    using Piece = std::conditional_t<(DPV * sizeof(T)) % 16 == 0, uint4, uint2>;
    constexpr int NPC = (int)(DPV * sizeof(T) / sizeof(Piece));
    for (int kk0 = rg; kk0 < nk; kk0 += kVRows * RPI) {
      Piece raw[kVRows][NPC];
#pragma unroll
      for (int u = 0; u < kVRows; ++u) {
        const int kk = kk0 + u * RPI < nk ? kk0 + u * RPI : rg;
        const int64_t r = lo + kk;
        const Piece* src = reinterpret_cast<const Piece*>((r == n ? vnew : vbase + r * D) + dl);
#pragma unroll
        for (int x = 0; x < NPC; ++x) {
          if constexpr (sizeof(Piece) == 16) raw[u][x] = load16_nt(src + x);  // streamed: read once per step
          else raw[u][x] = src[x];
        }
      }
#pragma unroll
      for (int u = 0; u < kVRows; ++u) {
        const int kk = kk0 + u * RPI;
        if (kk < nk) {
          float vv[DPV];
          load_vec<T, DPV>(reinterpret_cast<const T*>(raw[u]), vv);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pg = s_p[w][kk][g];
#pragma unroll
            for (int e = 0; e < DPV; ++e) acc_o[g][e] = fmaf(pg, vv[e], acc_o[g][e]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < DPV; ++e)
#pragma unroll
        for (int o = LPR; o < kWave; o <<= 1) acc_o[g][e] += __shfl_xor(acc_o[g][e], o);
    if (rg == 0)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < DPV; ++e) s_o[(w * G + g) * D + dl + e] += acc_o[g][e];
    wave_sync();
  }
  __syncthreads();
  T* out = static_cast<T*>(a.o) + ((int64_t)s * a.Hq + h * G) * D;
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int g = i / D;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += s_o[ww * G * D + i];
    store1<T>(out + i, s_L[g] > 0.f ? v / s_L[g] : 0.f);
  }
}

__global__ void decode_bump_kernel(int32_t* len, int32_t S, int64_t cap) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S && len[s] >= 0 && len[s] < cap) len[s] += 1;
}

hipError_t launch_decode(const DecodeArgs& d, void* k_cache, void* v_cache, float* pyr, int32_t* len,
                         const void* q_new, const void* k_new, const void* v_new, void* o, int32_t* idx,
                         float* score, int32_t* err, hipStream_t stream) {
  if (d.K > 32 || d.C > 128) return hipErrorInvalidValue;
  const int64_t plane = (int64_t)d.S * d.Hkv * d.geo.rows * d.D;
  _Float16* f16 = reinterpret_cast<_Float16*>(pyr + plane);
  DecodeKArgs a{k_cache, v_cache, pyr, f16, reinterpret_cast<int32_t*>(f16 + plane), len, q_new, k_new, v_new, o, idx,
                score, err, d.S, d.Hq, d.Hkv, d.C, d.K, d.cap, d.scale, d.geo};
  const dim3 grid((unsigned)((int64_t)d.S * d.Hkv));
  hipError_t e = dispatch_tdg(d.dtype, d.D, d.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    constexpr int NW = G >= 8 ? 4 : 8;
    if (d.C <= 32)
      PISA_LAUNCH("decode", stream, (decode_kernel<T, D, G, NW, 2>), grid, dim3(NW * kWave), 0, a);
    else if (d.C <= 64)
      PISA_LAUNCH("decode", stream, (decode_kernel<T, D, G, NW, 4>), grid, dim3(NW * kWave), 0, a);
    else
      PISA_LAUNCH("decode", stream, (decode_kernel<T, D, G, NW, 8>), grid, dim3(NW * kWave), 0, a);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  PISA_LAUNCH("decode_bump", stream, decode_bump_kernel, dim3((d.S + 255) / 256), dim3(256), 0, len, d.S, d.cap);
  return hipGetLastError();
}

}  // namespace pisa
