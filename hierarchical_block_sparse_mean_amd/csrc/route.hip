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
  unsigned long long* counts;  // optional work counters (diagnostics), or null
  const void* q;
  const void* k;
  const float* pyr;
  const _Float16* f16;  // block-floating-point copy of the summaries
  const int32_t* ex;
  int32_t* idx;
  float* score;
  int32_t B, N, Hq, Hkv, C, K, L;
  int32_t causal;
  int64_t cap;
  float scale;
  PyrGeom geo;
  // stage 1: levels stage_level..stage_top of the fp16 summaries (stage_rows
  // rows from row stage_off of a head) sit in LDS; chunks workgroups per (b, h)
  int32_t stage_level, stage_top, stage_rows;
  int64_t stage_off;
  int32_t chunks;
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

// ---- stage 1 on MFMA (bf16 inputs) -------------------------------------------
// Scores of the candidates of level l: q_h' . P_{l-1}[r] for the <= 2 nA
// child rows r, as (16 child rows) x d x (16 columns = the G_Q query heads)
// v_mfma_f32_16x16x32_f16 tiles.  Rows come from the pyramid's fp16
// block-floating-point copy (row * 2^-ex[row]); q is bf16, so q * 2^-eq is
// exact in fp16; the logit in log2 units is acc * 2^(ex + eq) * scale*log2e.
// A row costs d * 2 bytes of gather (half the fp32 row).  The sibling LSE is
// in-lane (accumulator rows 2c, 2c+1) and the GQA sum a shuffle over the G_Q
// columns.
// hb / xb: the rows (pitch PITCH elements) and exponents of a head, in LDS
// or in global memory; lvl: the child level's first row there.
// GATHER (rows in global memory, pitch D): a row tile is gathered as
// 128-byte pieces, eight lanes per piece and eight rows per load (a load in
// the MFMA operand layout, sixteen rows of 64 bytes, is served about three
// times slower from L2), written to the wave's LDS tile (16 rows, pitch
// PITCH) and read back in the operand layout.
// Only G_Q of a tile's 16 columns carry query heads, so the results of
// P = 16 / max(G_Q, 4) consecutive row tiles are packed into one accumulator
// set (tile p's useful columns moved into lane bank(s) p by DPP row shifts)
// before the scaling, the sibling LSE and the GQA sum, which then run once
// per P tiles on lanes that all carry data.
template <int D, int G, int PITCH, bool GATHER>
__device__ __forceinline__ void score_level_mfma(RouteLds& s, int nA, const halfx8* fq, int eq_p, const _Float16* hb,
                                                 const int32_t* xb, int32_t lvl, int32_t m_child, int32_t tl,
                                                 float sl2, int64_t* rows_out, _Float16* tile) {
  constexpr int NS = D / 32;
  constexpr int GP = G < 4 ? 4 : G;  // lanes per packed tile
  constexpr int P = 16 / GP;         // tiles per packed set
  const int lane = lane_id(), g = lane >> 4, col = lane & 15;
  const int qp = col / GP, hc = col % GP;  // packed: tile qp of the set, head hc
  const int nt = (2 * nA + 15) >> 4;      // row tiles of this level
  // gathers of row tile rtg into gv: rows (lane / 8) + 8 (st % 2) of the
  // tile, elements [64 (st / 2) + 8 (lane % 8), + 8)
  auto gather = [&](int rtg, halfx8* gv) {
    const int row_a = 16 * rtg + (lane >> 3), row_b = row_a + 8;
    int32_t ca = s.cand[(row_a >> 1) & (kWave - 1)], cb = s.cand[(row_b >> 1) & (kWave - 1)];
    asm volatile("" : "+v"(ca), "+v"(cb));
    const int32_t ra = ((row_a >> 1) < nA) ? 2 * ca + (row_a & 1) : 0x7fffffff;
    const int32_t rb = ((row_b >> 1) < nA) ? 2 * cb + (row_b & 1) : 0x7fffffff;
    const uint32_t rra = (uint32_t)(lvl + ((ra < m_child && ra <= tl) ? ra : 0));
    const uint32_t rrb = (uint32_t)(lvl + ((rb < m_child && rb <= tl) ? rb : 0));
#pragma unroll
    for (int st = 0; st < NS; ++st)
      gv[st] = *reinterpret_cast<const halfx8*>(hb + ((st & 1) ? rrb : rra) * (uint32_t)D + 64 * (st >> 1) +
                                                8 * (lane & 7));
  };
  for (int rt0 = 0; rt0 < nt; rt0 += P) {
    floatx4 acc[P];
    halfx8 gv_next[NS];
    // the gathers are issued at a raised wave priority, so that the SIMD's
    // other waves (sorting, scoring) do not delay the level's critical loads
    // (stage 1 at 128K: 5.13 -> 5.05 ms)
    if constexpr (GATHER) {
      __builtin_amdgcn_s_setprio(2);
      gather(rt0, gv_next);
      __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
      // A row `col` of tile rt: child (row & 1) of candidate row >> 1; an
      // invalid row (or a tile past the last) reads row 0 of the level
      // (finite data) and gets scale 0 and bias -inf below.  Offsets within
      // a head fit 32 bits.
      // (rows < 64: candidate reads stay inside s.cand and need no branch)
      const int rt = rt0 + q;
      const int row = 16 * rt + col;
      const int c = row >> 1;
      int32_t cv = s.cand[c & (kWave - 1)];
      asm volatile("" : "+v"(cv));  // read unconditionally (not sunk into a branch)
      const int32_t r = (c < nA) ? 2 * cv + (row & 1) : 0x7fffffff;
      const bool vrow = r < m_child && r <= tl;  // exists and starts at or before t
      if (rows_out != nullptr && rt < nt) *rows_out += __popcll(__ballot(vrow) & 0xFFFFull);
      const uint32_t rr = (uint32_t)(lvl + (vrow ? r : 0));
      const int32_t er = xb[rr];
      // step st covers elements [32 st, 32 st + 32): the four lane groups
      // read one contiguous 64-byte span of the row per load.  All NS loads
      // are issued before the first product (the barrier keeps the
      // scheduler from sinking each load next to its use).
      halfx8 fa[NS];
      if constexpr (GATHER) {
        // this tile's rows arrived in gv_next; the next tile's loads are
        // issued before they are stored, so two tiles are in flight
        halfx8 gv[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) gv[st] = gv_next[st];
        if (q + 1 < P) {
          __builtin_amdgcn_s_setprio(2);
          gather(rt + 1, gv_next);
          __builtin_amdgcn_s_setprio(0);
        }
#pragma unroll
        for (int st = 0; st < NS; ++st)
          *reinterpret_cast<halfx8*>(tile + ((lane >> 3) + 8 * (st & 1)) * PITCH + 64 * (st >> 1) + 8 * (lane & 7)) =
              gv[st];
        wave_sync();
#pragma unroll
        for (int st = 0; st < NS; ++st) fa[st] = *reinterpret_cast<const halfx8*>(tile + col * PITCH + 32 * st + 8 * g);
      } else {
#pragma unroll
        for (int st = 0; st < NS; ++st)
          fa[st] = *reinterpret_cast<const halfx8*>(hb + rr * (uint32_t)PITCH + 32 * st + 8 * g);
      }
      __builtin_amdgcn_sched_barrier(0);
      acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st) acc[q] = mma16x16x32(fa[st], fq[st], acc[q]);
      // (scale, bias) of row 16 q + col: (2^ex * scale*log2e, 0), or (0, -inf)
      // for a missing child
      if (g == 0) s.fb[16 * q + col] = vrow ? float2{ldexpf(sl2, er), 0.f} : float2{0.f, -INFINITY};
    }
    // pack: lane bank(s) of tile q take tile q's columns 0..GP-1
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[0][i];
      if constexpr (P >= 2)
        v = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(acc[1][i]), 0x110 + GP,
                                                       0xF, P == 2 ? 0xC : 0x2, false));
      if constexpr (P == 4) {
        v = __int_as_float(
            __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(acc[2][i]), 0x118, 0xF, 0x4, false));
        v = __int_as_float(
            __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(acc[3][i]), 0x11C, 0xF, 0x8, false));
      }
      x[i] = v;
    }
    wave_sync();
    // rows 16 qp + 4 g + i of the set, head hc: logits in log2 units
    const float4 fb01 = *reinterpret_cast<const float4*>(&s.fb[16 * qp + 4 * g]);
    const float4 fb23 = *reinterpret_cast<const float4*>(&s.fb[16 * qp + 4 * g + 2]);
    wave_sync();  // s.fb is rewritten by the next set
    const float x0 = fmaf(ldexpf(x[0], eq_p), fb01.x, fb01.y), x1 = fmaf(ldexpf(x[1], eq_p), fb01.z, fb01.w);
    const float x2 = fmaf(ldexpf(x[2], eq_p), fb23.x, fb23.y), x3 = fmaf(ldexpf(x[3], eq_p), fb23.z, fb23.w);
    // sibling LSE: max + log2(1 + 2^-|a - b|).  Child 0 of a candidate always
    // exists, so a stored score is finite; a missing child 1 (-inf) adds 0.
    float u0 = fmaxf(x0, x1) + __log2f(1.f + exp2_nonpos(-fabsf(x0 - x1)));
    float u1 = fmaxf(x2, x3) + __log2f(1.f + exp2_nonpos(-fabsf(x2 - x3)));
    u0 = lane_group_sum<G>(u0);
    u1 = lane_group_sum<G>(u1);
    const int c0 = 8 * (rt0 + qp) + 2 * g;
    if (hc == 0 && rt0 + qp < nt) {
      if (c0 < nA) s.score[c0] = u0;
      if (c0 + 1 < nA) s.score[c0 + 1] = u1;
    }
  }
}

// KP: K when K is 16 or 32 (top-K by half sorts), else 0 (full wave sort).
// CNT: a separate instance that also accumulates the work counters.
// Persistent workgroups of kRouteWgWaves waves, chunks of them per (b, h):
// the workgroup first copies the coarse levels of its head's fp16 summaries
// (every level from stage_level up, rows padded by 16 bytes so that the 16
// rows of a fragment read fall in different LDS banks) into LDS, where every
// query of the head finds them; each wave then routes the queries
// t = chunk W + w, + chunks W, ... (W = waves).  Levels whose children are
// staged read them from LDS, the finer levels gather from global memory.
constexpr int kRouteWgWaves = 16;

template <int D>
constexpr int stage_pitch() { return D + 8; }  // fp16 elements per staged row

template <int D, int G, int KP, bool CNT>
__global__ __launch_bounds__(kRouteWgWaves* kWave) PISA_MFMA_REGS void route_mfma_kernel(RouteArgs a) {
  constexpr int NS = D / 32;
  constexpr int SP = stage_pitch<D>();
  constexpr float kLog2e = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ RouteLds s_r[kRouteWgWaves];
  // each wave's tile of 16 gathered rows (levels below the LDS stage)
  __shared__ __align__(16) _Float16 s_tile[kRouteWgWaves][16 * SP];
  _Float16* s_rows = reinterpret_cast<_Float16*>(smem_raw);                             // [stage_rows][SP]
  int32_t* s_exs = reinterpret_cast<int32_t*>(smem_raw + (size_t)a.stage_rows * SP * 2);  // [stage_rows]
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % a.Hkv);
  const int64_t rb = bid / a.Hkv;
  const int b = (int)(rb % a.B);
  const int chunk = (int)(rb / a.B);
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const _Float16* hb = a.f16 + bh * a.geo.rows * D;
  const int32_t* xb = a.ex + bh * a.geo.rows;
  for (int i = threadIdx.x; i < a.stage_rows * (D / 8); i += blockDim.x) {
    const int r = i / (D / 8), d = (i % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(s_rows + r * SP + d) = *reinterpret_cast<const uint4*>(hb + (a.stage_off + r) * D + d);
  }
  for (int i = threadIdx.x; i < a.stage_rows; i += blockDim.x) s_exs[i] = xb[a.stage_off + i];
  __syncthreads();  // the only workgroup barrier: the query loop below is per wave

  const int g = lane >> 4, col = lane & 15;
  RouteLds& s = s_r[w];
  const bool causal = a.causal != 0;
  const float sl2 = a.scale * kLog2e;
  // level sizes and the last valid block by shifts: M_l = ceil(M_1 / 2^(l-1))
  // and block j of level l starts at j C 2^(l-1) <= t iff j <= (t / C) >> (l-1)
  const int32_t M1 = (int32_t)level_rows(a.N, a.C, 1);
  const int64_t tstep = (int64_t)a.chunks * kRouteWgWaves;
  // diagnostics only: queries, scored candidates, rows, scored levels, kept
  // blocks of this wave, added to the counters once at the end
  unsigned long long w_q = 0, w_cands = 0, w_rows_sum = 0, w_levels = 0, w_kept = 0, w_rows_mem = 0;
  for (int64_t t = (int64_t)chunk * kRouteWgWaves + w; t < a.N; t += tstep) {
    // B operand: column col = query head col of the group (zero beyond G_Q),
    // scaled by 2^-eq into fp16 (exact for bf16 values)
    float qv[NS][8];
    float mx = 0.f;
    if (col < G) {
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.Hq + h * G + col) * a.N + t) * D;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        load8<uint16_t>(qrow + 32 * st + 8 * g, qv[st]);  // same element order as the rows
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
    // the exponent of head col % max(G, 4), the head a packed lane carries
    const int eq_p = __shfl(eq, col % (G < 4 ? 4 : G));
    halfx8 fq[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) fq[st][e] = to_f16_scaled(qv[st][e], eq);
    int nA = 1;
    wave_sync();  // the previous query's last reads of s are done
    if (lane == 0) s.cand[0] = 0;
    int32_t kept = (lane == 0) ? 0 : -1;
    int nI = 1;
    int64_t w_rows = 0, w_rows_lds = 0;  // diagnostics only
    int64_t* rows_ptr = CNT ? &w_rows : nullptr;
    int64_t* rows_lds_ptr = CNT ? &w_rows_lds : nullptr;
    wave_sync();
    const int32_t tc = (int32_t)t / a.C;
    for (int32_t l = a.L; l >= 2; --l) {
      // valid blocks of level l: index < M_l and (causal) first token <= t
      const int32_t ml = ((M1 - 1) >> (l - 1)) + 1;
      const int32_t tl_blk = causal ? (tc >> (l - 1)) : 0x7fffffff;
      const int32_t j = (lane < nA) ? s.cand[lane] : 0x7fffffff;
      const bool valid = j < ml && j <= tl_blk;
      const uint64_t mask = __ballot(valid);
      const int pos = __popcll(mask & ((1ull << lane) - 1ull));
      nA = __popcll(mask);
      wave_sync();
      if (valid) s.cand[pos] = j;
      wave_sync();
      if (nA > a.K) {
        const int32_t m_child = ((M1 - 1) >> (l - 2)) + 1;
        const int32_t tl = causal ? (tc >> (l - 2)) : 0x7fffffff;
        const int32_t lvl = (int32_t)a.geo.level_off[l - 1];
        if (l - 1 >= a.stage_level && l - 1 <= a.stage_top)
          score_level_mfma<D, G, SP, false>(s, nA, fq, eq_p, s_rows, s_exs, lvl - (int32_t)a.stage_off, m_child, tl,
                                            sl2, rows_lds_ptr, nullptr);
        else
          score_level_mfma<D, G, SP, true>(s, nA, fq, eq_p, hb, xb, lvl, m_child, tl, sl2, rows_ptr, s_tile[w]);
        w_cands += nA;
        w_levels += 1;
        wave_sync();
        uint64_t key = (lane < nA) ? score_key(s.score[lane], s.cand[lane]) : 0ull;
        if (KP) key = top_half<(KP ? KP : 16)>(key);
        else key = wave_sort_desc(key);
        nI = a.K;
        kept = (lane < nI) ? key_index(key) : -1;
      } else {
        nI = nA;
        kept = (lane < nA) ? s.cand[lane] : -1;
      }
      if (l > 2) {
        wave_sync();
        if (lane < nI) {
          s.cand[2 * lane] = 2 * kept;
          s.cand[2 * lane + 1] = 2 * kept + 1;
        }
        nA = 2 * nI;
        wave_sync();
      }
    }
    uint64_t k2 = (lane < nI) ? index_key(kept, 0.f) : 0ull;
    if (KP) k2 = group_sort_desc<(KP ? KP : 16)>(k2);
    else k2 = wave_sort_desc(k2);
    if (lane < a.K) a.idx[(bh * a.N + t) * a.K + lane] = (lane < nI) ? index_key_index(k2) : -1;
    if (CNT) {
      w_q += 1;
      w_rows_sum += (unsigned long long)(w_rows + w_rows_lds);
      w_rows_mem += (unsigned long long)w_rows;
      w_kept += (unsigned long long)nI;
    }
  }
  if (CNT && lane == 0) {
    atomicAdd(&a.counts[0], w_q);
    atomicAdd(&a.counts[1], w_cands);
    atomicAdd(&a.counts[2], w_rows_sum);
    atomicAdd(&a.counts[5], w_rows_mem);
    atomicAdd(&a.counts[3], w_levels);
    atomicAdd(&a.counts[4], w_kept);
  }
}

// Staged levels for stage 1: the coarsest levels of a head whose rows fit a
// 144 KB LDS budget (the whole pyramid for short sequences), one workgroup
// per compute unit (two with half the budget each were slower: the finer
// levels gathered from memory cost more than the extra waves gain).
static void route_stage_plan(const Problem& p, RouteArgs& a, size_t& lds) {
  constexpr int wg_per_cu = 1;
  const size_t pitch_bytes = (size_t)(p.D + 8) * 2 + 4;  // padded fp16 row + exponent
  // 160 KB per CU less the waves' candidate lists (1 KB each) and their
  // gather tiles (16 rows of (D + 8) fp16 each)
  const size_t budget = (size_t)160 * 1024 - (size_t)kRouteWgWaves * (1024 + 16 * (p.D + 8) * 2);
  a.stage_level = p.geo.levels_cap + 1;
  a.stage_top = p.geo.levels_cap;
  a.stage_rows = 0;
  a.stage_off = p.geo.rows;
  // (staging only the finest level that fits instead was slower: the coarse
  // levels are read by every query of the head)
  for (int32_t l = 1; l <= p.geo.levels_cap; ++l) {
    const int64_t rows = p.geo.rows - p.geo.level_off[l];
    if ((size_t)rows * pitch_bytes <= budget) {
      a.stage_level = l;
      a.stage_rows = (int32_t)rows;
      a.stage_off = p.geo.level_off[l];
      break;
    }
  }
  lds = (size_t)a.stage_rows * pitch_bytes;
  // workgroups: about wg_per_cu per compute unit over all (b, h)
  const int64_t heads = (int64_t)p.B * p.Hkv;
  const int64_t want = (256 * (int64_t)wg_per_cu + heads - 1) / heads;
  const int64_t most = (p.N + kRouteWgWaves - 1) / kRouteWgWaves;
  a.chunks = (int32_t)(want < 1 ? 1 : (want > most ? most : want));
}

hipError_t launch_route(const Problem& p, const void* q, const void* k, const float* pyr, int32_t* idx,
                        float* score, bool fused, hipStream_t stream, unsigned long long* counts) {
  const int64_t plane = (int64_t)p.B * p.Hkv * p.geo.rows * p.D;
  const _Float16* f16 = reinterpret_cast<const _Float16*>(pyr + plane);
  RouteArgs a{counts, q, k, pyr, f16, reinterpret_cast<const int32_t*>(f16 + plane), idx, score, p.B, p.N, p.Hq, p.Hkv, p.C, p.K, p.L, p.causal ? 1 : 0,
              p.cap, p.scale, p.geo, 0, 0, 0, 0, 1};
  const int64_t blocks = (int64_t)p.B * p.Hkv * ((p.N + kRouteWaves - 1) / kRouteWaves);
  return dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    constexpr int G = decltype(gc)::value;
    if (fused)
      PISA_LAUNCH("route_fused", stream, (route_kernel<T, D, G, true>), dim3((unsigned)blocks),
                  dim3(kRouteWaves * kWave), 0, a);
    else if (std::is_same<T, uint16_t>::value) {
      RouteArgs ra = a;
      size_t lds = 0;
      route_stage_plan(p, ra, lds);
      const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * ra.chunks)), block(kRouteWgWaves * kWave);
      auto run = [&](auto kern) -> hipError_t {
        if (lds > 65536) {
          hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (e != hipSuccess) return e;
        }
        PISA_LAUNCH(counts ? "route_stage1_counted" : "route_stage1", stream, kern, grid, block, lds, ra);
        return hipSuccess;
      };
      hipError_t e;
      if (p.K == 16) e = counts ? run(route_mfma_kernel<D, G, 16, true>) : run(route_mfma_kernel<D, G, 16, false>);
      else if (p.K == 32) e = counts ? run(route_mfma_kernel<D, G, 32, true>) : run(route_mfma_kernel<D, G, 32, false>);
      else e = counts ? run(route_mfma_kernel<D, G, 0, true>) : run(route_mfma_kernel<D, G, 0, false>);
      if (e != hipSuccess) return e;
    }
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
