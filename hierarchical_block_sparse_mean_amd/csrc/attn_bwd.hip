// Backward of the block-sparse attention ("Block Sparse Attention with
// Log-Linear Complexity", hyper.ai page, section "block-sparse attention", the
// o_t equation; the page names training kernels but gives no backward, so
// this is the calculus of that equation over a fixed selection: the selection
// is index-valued and carries no gradient).  With p = softmax(z),
// z_i = q_t . k_i * scale over the keys of the kept leaves (i <= t causally)
// and L = sum_t dO_t . o_t:
//   D_t = dO_t . o_t,  dP_i = dO_t . v_i,  dS_i = p_i (dP_i - D_t),
//   dq_t = scale sum_i dS_i k_i,  dk_i += scale dS_i q_t,  dv_i += p_i dO_t.
//
// Leaf-major, like the forward: the kept (query, leaf) pairs are clustered by
// leaf; a workgroup holds the leaf's K, V and K^T in LDS and walks its query
// tiles (16 columns = 16/G_Q queries x G_Q heads), all waves on one round of
// tiles (two tiles for 16-bit inputs, one for fp32) between barriers:
//   phase A (waves split the (16-key block, tile) items): S^T = K Q^T and
//     dP^T = V dO^T on MFMA, p = exp(z - lse) from the forward's lse,
//     dS = p (dP - D), both written to LDS;
//   phase B (waves split the 16-dim blocks): dV^T += dO^T P and dK^T += Q^T dS
//     (16x16x16 MFMA over the tile's columns, accumulated in registers across
//     tiles), and dQ^T = K^T dS^T (16x16x32 MFMA over the keys) written as a
//     partial per (query, slot, head).
// At the end of its chunk a workgroup adds its dK, dV sums into fp32
// accumulators (atomics: a leaf's queries may span several chunks); a merge
// kernel sums each query's K partial dQ rows, a last pass converts dK, dV.
#include "kernels.h"

namespace pisa {

// waves per workgroup: 8 when a leaf tile fills most of the LDS (C > 64) and
// d has a 16-dim block per wave, so that one resident workgroup still keeps
// 8 waves in flight; 4 otherwise
template <int D, int NKB>
constexpr int bwd_waves() { return NKB >= 8 && D >= 128 ? 8 : 4; }
// (query, slot) pairs per workgroup: a chunk stages its leaf's K, V and K^T
// once and adds its dK, dV sums with atomics once; 1024 for leaves of more
// than 64 keys (8 key blocks), 256 otherwise, where the pair codes' LDS would
// cost the second resident workgroup (measured best per leaf size)
template <int NKB>
constexpr int bwd_chunk_max() { return NKB >= 8 ? 1024 : 256; }
static int bwd_chunk(const Problem& p) { return p.C > 64 ? 1024 : 256; }
constexpr size_t kBwdBudget = (size_t)24 << 30;  // partial dQ rows per head chunk

static size_t b256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  int64_t heads, M1, Mb, ncl, slots, max_chunks;  // Mb: cluster bins per head
  size_t off_counts, off_cursor, off_offsets, off_chunks, off_map, off_pairs, off_dq, off_hist, off_rowdot, off_dk,
      off_dv, total;
};

static BwdLayout bwd_layout(const Problem& p) {
  BwdLayout L{};
  L.M1 = level_rows(p.N, p.C, 1);
  L.Mb = cluster_bins(p.N, L.M1, kAttnBins);
  const size_t esz = p.dtype == 1 ? 2 : 4;  // partial dQ rows in the input dtype
  const size_t per_head = (size_t)p.N * p.K * (4 + (size_t)p.G * p.D * esz) + (size_t)L.Mb * 16;
  const int64_t BH = (int64_t)p.B * p.Hkv;
  int64_t hmax = (int64_t)(kBwdBudget / per_head);
  if (hmax < 1) hmax = 1;
  if (hmax > BH) hmax = BH;
  const int64_t nchunks = (BH + hmax - 1) / hmax;
  L.heads = (BH + nchunks - 1) / nchunks;
  L.ncl = L.heads * L.Mb;
  L.slots = L.heads * (int64_t)p.N * p.K;
  L.max_chunks = (L.slots + bwd_chunk(p) - 1) / bwd_chunk(p) + L.ncl;
  size_t off = 0;
  L.off_counts = off;
  off = b256(off + 4 * (size_t)L.ncl);
  L.off_cursor = off;
  off = b256(off + 4 * (size_t)L.ncl);
  L.off_offsets = off;
  off = b256(off + 4 * (size_t)(L.ncl + 1));
  L.off_chunks = off;
  off = b256(off + 4 * (size_t)(L.ncl + 1));
  L.off_map = off;
  off = b256(off + sizeof(ChunkEntry) * (size_t)L.max_chunks);
  L.off_pairs = off;
  off = b256(off + 4 * (size_t)L.slots);
  L.off_dq = off;
  off = b256(off + esz * (size_t)L.slots * p.G * p.D);
  L.off_hist = off;
  off = b256(off + cluster_scratch_bytes(L.heads, (int64_t)p.N * p.K, L.Mb));
  L.off_rowdot = off;
  off = b256(off + 4 * (size_t)p.B * p.Hq * p.N);
  L.off_dk = off;
  off = b256(off + 4 * (size_t)BH * p.N * p.D);
  L.off_dv = off;
  off = b256(off + 4 * (size_t)BH * p.N * p.D);
  L.total = off;
  return L;
}

size_t attn_bwd_workspace_bytes(const Problem& p) { return bwd_layout(p).total; }

// ---- D_t = dO_t . o_t per (b, query head, t) ----------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ dout, const T* __restrict__ o, int64_t rows,
                                                     float* __restrict__ rowdot) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    float x[8], y[8];
    load8<T>(dout + row * D + sub * 8, x);
    load8<T>(o + row * D + sub * 8, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(x[e], y[e], s);
  }
  s = group_sum<LPR>(s);
  if (row < rows && sub == 0) rowdot[row] = s;
}

// ---- 16x16x16 MFMA: lane group g supplies contraction elements 4g .. 4g+3 ----
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ floatx4 mma16(const float* a4, const float* b4, floatx4 acc, uint16_t) {
  const uint2 ua = {pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3])};
  const uint2 ub = {pack_bf16x2(b4[0], b4[1]), pack_bf16x2(b4[2], b4[3])};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, ua), __builtin_bit_cast(shortx4, ub),
                                                  acc, 0, 0, 0);
}
// B given as four bf16 values (raw bits, 8 bytes)
__device__ __forceinline__ floatx4 mma16_braw(const float* a4, uint2 b4, floatx4 acc) {
  const uint2 ua = {pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3])};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, ua), __builtin_bit_cast(shortx4, b4),
                                                  acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(const float* a4, const float* b4, floatx4 acc, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[i], b4[i], acc, 0, 0, 0);
  return acc;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* rowdot;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* chunk_off;
  const ChunkEntry* chunk_map;  // work chunk -> (cluster, first pair, pairs)
  const int32_t* pairs;
  void* dq_part;  // [heads][N][K][G][D], input dtype
  float* dk_acc;   // [B][Hkv][N][D]
  float* dv_acc;
  int64_t ncl, M1, Mb, head0;
  int32_t N, Hq, Hkv, C, K;
  int32_t chunk;  // pairs per work chunk
  int32_t causal;
  int64_t cap;
  float scale;
};

template <typename T, int D, int G, int NKB>
__global__ __launch_bounds__((bwd_waves<D, NKB>() * kWave)) PISA_MFMA_REGS void attn_bwd_kernel(BwdArgs a) {
  constexpr int NW = bwd_waves<D, NKB>();
  constexpr int NS = D / 32;
  constexpr int TQ = 16 / G;
  constexpr int CP = NKB * 16;
  constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int KP = D + EPV;               // row pitch of K, V, q, dO tiles
  constexpr int TP = CP + EPV;              // row pitch of K^T
  constexpr int NDB = D / 16;
  constexpr int DBW = NDB / NW;  // dim blocks per wave
  static_assert(DBW >= 1 && NDB % NW == 0, "every wave owns whole 16-dim blocks");
  constexpr float kLog2e = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* s_k = reinterpret_cast<T*>(smem_raw);  // [CP][KP]
  T* s_v = s_k + CP * KP;                    // [CP][KP]
  T* s_kt = s_v + CP * KP;                   // [D][TP]
  // RT tiles of 16 columns per round of barriers: two for 16-bit inputs,
  // whose p and dS are staged in bf16 (the rounding the MFMA operands apply
  // anyway), one for fp32 inputs (fp32 staging)
  constexpr bool B16 = sizeof(T) == 2;
  constexpr int RT = B16 ? 2 : 1;
  constexpr int NC = 16 * RT;  // columns per round
  constexpr int PPITCH = NC + 4;  // p / dS row pitch (elements): conflict-free 8/16-byte reads
  using PT = std::conditional_t<B16, uint16_t, float>;
  __shared__ __align__(16) T s_q[NC][KP];    // the round's query rows, one per column
  __shared__ __align__(16) T s_do[NC][KP];   // and their output gradients
  __shared__ __align__(16) PT s_p[CP][PPITCH];
  __shared__ __align__(16) PT s_ds[CP][PPITCH];
  __shared__ float s_lse[NC], s_rd[NC];
  __shared__ int32_t s_pr[NC];
  __shared__ int32_t s_cpr[bwd_chunk_max<NKB>()];  // the chunk's pair codes

  const ChunkEntry ce = a.chunk_map[blockIdx.x];
  if (ce.cluster < 0) return;  // past the last work chunk (uniform over the workgroup)
  const int64_t c = ce.cluster;
  const int64_t hl = c / a.Mb;
  const int64_t j = c % a.M1;
  const int64_t bh = a.head0 + hl;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int64_t p_begin = ce.begin;
  const int64_t p_end = p_begin + ce.count;

  const int64_t key0 = j * (int64_t)a.C;
  const int nkeys = (int)((a.N - key0) < a.C ? (a.N - key0) : a.C);
  const T* kh = static_cast<const T*>(a.k) + bh * a.cap * D;
  const T* vh = static_cast<const T*>(a.v) + bh * a.cap * D;
  for (int i = threadIdx.x; i < CP * (D / EPV); i += blockDim.x) {
    const int r = i / (D / EPV), d = (i % (D / EPV)) * EPV;
    uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (r < nkeys) {
      kv = *reinterpret_cast<const uint4*>(kh + (key0 + r) * D + d);
      vv = *reinterpret_cast<const uint4*>(vh + (key0 + r) * D + d);
    }
    *reinterpret_cast<uint4*>(s_k + r * KP + d) = kv;
    *reinterpret_cast<uint4*>(s_v + r * KP + d) = vv;
    const T* ke = reinterpret_cast<const T*>(&kv);
#pragma unroll
    for (int e = 0; e < EPV; ++e) s_kt[(d + e) * TP + r] = ke[e];
  }
  for (int i = threadIdx.x; i < bwd_chunk_max<NKB>(); i += blockDim.x)
    s_cpr[i] = p_begin + i < p_end ? a.pairs[p_begin + i] : -1;
  __syncthreads();
  const int n = (int)(p_end - p_begin);

  const int w = threadIdx.x / kWave, lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const float sl2 = a.scale * kLog2e;
  const T* qb = static_cast<const T*>(a.q);
  const T* gb = static_cast<const T*>(a.dout);
  floatx4 dvt[DBW][NKB], dkt[DBW][NKB];
#pragma unroll
  for (int di = 0; di < DBW; ++di)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      dvt[di][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      dkt[di][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  // a round's staging work: NC columns x D / EPV 16-byte pieces of q and dO
  // (column cc = query cc / G of the round x head cc % G), plus lse and D_t of
  // the columns; each thread fetches its share of the next round into
  // registers while the current round is computed
  constexpr int PIECES = NC * (D / EPV);
  constexpr int PPT = (PIECES + NW * kWave - 1) / (NW * kWave);  // pieces per thread
  uint4 nq[PPT], ng[PPT];
  float nlse = 0.f, nrd = 0.f;
  int32_t npr = -1;
  auto fetch = [&](int i0) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int i = threadIdx.x + k * NW * kWave;
      nq[k] = uint4{0u, 0u, 0u, 0u};
      ng[k] = uint4{0u, 0u, 0u, 0u};
      if (i < PIECES) {
        const int cc = i / (D / EPV), d = (i % (D / EPV)) * EPV;
        const int jj = i0 + cc / G;
        const int32_t pr = jj < n ? s_cpr[jj] : -1;
        if (pr >= 0) {
          const int64_t row = ((int64_t)b * a.Hq + h * G + cc % G) * a.N + (pr >> 5);
          nq[k] = *reinterpret_cast<const uint4*>(qb + row * D + d);
          ng[k] = *reinterpret_cast<const uint4*>(gb + row * D + d);
        }
      }
    }
    if (threadIdx.x < NC) {
      const int cc = threadIdx.x;
      const int jj = i0 + cc / G;
      npr = jj < n ? s_cpr[jj] : -1;
      const int64_t row = ((int64_t)b * a.Hq + h * G + cc % G) * a.N + (npr >= 0 ? (npr >> 5) : 0);
      nlse = npr >= 0 ? a.lse[row] : 0.f;
      nrd = npr >= 0 ? a.rowdot[row] : 0.f;
    }
  };
  auto to_pt = [](float x) -> PT {
    if constexpr (B16) return f32_to_bf16(x);
    else return x;
  };
  auto from_pt = [](PT x) -> float {
    if constexpr (B16) return bf16_to_f32(x);
    else return x;
  };
  if (n > 0) fetch(0);
  for (int i0 = 0; i0 < n; i0 += TQ * RT) {
    // stage the fetched round
    if (threadIdx.x < NC) {
      s_pr[threadIdx.x] = npr;
      s_lse[threadIdx.x] = nlse;
      s_rd[threadIdx.x] = nrd;
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int i = threadIdx.x + k * NW * kWave;
      if (i < PIECES) {
        const int cc = i / (D / EPV), d = (i % (D / EPV)) * EPV;
        *reinterpret_cast<uint4*>(&s_q[cc][d]) = nq[k];
        *reinterpret_cast<uint4*>(&s_do[cc][d]) = ng[k];
      }
    }
    __syncthreads();
    if (i0 + TQ * RT < n) fetch(i0 + TQ * RT);  // the next round's rows, in flight during this one
    // phase A: (key block, tile) items of this wave
    for (int item = w; item < NKB * RT; item += NW) {
      const int kb = item % NKB, tt = item / NKB;
      const int cc = tt * 16 + col;
      Frag<T> fq[NS], fg[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        fq[s].load(&s_q[cc][g * (D / 4) + 8 * s]);
        fg[s].load(&s_do[cc][g * (D / 4) + 8 * s]);
      }
      const int32_t prc = s_pr[cc];
      int lim = 0;
      if (prc >= 0) {
        const int64_t t = prc >> 5;
        lim = a.causal ? (int)((t - key0 + 1) < nkeys ? (t - key0 + 1) : nkeys) : nkeys;
      }
      const float lse2 = s_lse[cc] * kLog2e, rd = s_rd[cc];
      floatx4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Frag<T> fk, fv;
        fk.load(s_k + (kb * 16 + col) * KP + g * (D / 4) + 8 * s);
        fv.load(s_v + (kb * 16 + col) * KP + g * (D / 4) + 8 * s);
        st = mma(fk, fq[s], st);
        dpt = mma(fv, fg[s], dpt);
      }
      // lane (g, col): keys kb*16 + 4g + i of column cc
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb * 16 + 4 * g + i;
        const float pv = key < lim ? exp2_nonpos(fminf(fmaf(st[i], sl2, -lse2), 0.f)) : 0.f;
        s_p[key][cc] = to_pt(pv);
        s_ds[key][cc] = to_pt(pv * (dpt[i] - rd));
      }
    }
    __syncthreads();
    // phase B: dim blocks of this wave, over the round's tiles
#pragma unroll
    for (int di = 0; di < DBW; ++di) {
      const int db = w * DBW + di;
      const int dim = db * 16 + col;  // A row of this lane
      float ag[RT][4], aq[RT][4];
#pragma unroll
      for (int tt = 0; tt < RT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ag[tt][e] = load1<T>(&s_do[tt * 16 + 4 * g + e][dim]);
          aq[tt][e] = load1<T>(&s_q[tt * 16 + 4 * g + e][dim]);
        }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tt = 0; tt < RT; ++tt) {
          if constexpr (B16) {
            const uint2 pp = *reinterpret_cast<const uint2*>(&s_p[kb * 16 + col][tt * 16 + 4 * g]);
            const uint2 dd = *reinterpret_cast<const uint2*>(&s_ds[kb * 16 + col][tt * 16 + 4 * g]);
            dvt[di][kb] = mma16_braw(ag[tt], pp, dvt[di][kb]);
            dkt[di][kb] = mma16_braw(aq[tt], dd, dkt[di][kb]);
          } else {
            const float4 pp = *reinterpret_cast<const float4*>(&s_p[kb * 16 + col][tt * 16 + 4 * g]);
            const float4 dd = *reinterpret_cast<const float4*>(&s_ds[kb * 16 + col][tt * 16 + 4 * g]);
            const float bp[4] = {pp.x, pp.y, pp.z, pp.w};
            const float bd[4] = {dd.x, dd.y, dd.z, dd.w};
            dvt[di][kb] = mma16(ag[tt], bp, dvt[di][kb], T{});
            dkt[di][kb] = mma16(aq[tt], bd, dkt[di][kb], T{});
          }
        }
      // dQ^T for these 16 dims and each tile: K^T (dims x keys) times dS^T
      // (keys x columns)
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
        const int cc = tt * 16 + col;
        floatx4 dqt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < CP / 32; ++ks) {
          Frag<T> fa, fb;
          fa.load(s_kt + dim * TP + ks * 32 + g * 8);
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = from_pt(s_ds[ks * 32 + g * 8 + e][cc]);
          fb.set(x);
          dqt = mma(fa, fb, dqt);
        }
        // lane (g, col): dims db*16 + 4g + i of column cc
        const int32_t pc = s_pr[cc];
        if (pc >= 0) {
          const int64_t rec = ((hl * a.N + (pc >> 5)) * a.K + (pc & 31)) * G + (col % G);
          T* dst = static_cast<T*>(a.dq_part) + rec * D + db * 16 + 4 * g;
          // (streaming stores: each partial row is read once, by the merge)
          if constexpr (B16) {
            store8_nt(dst, uint2{pack_bf16x2(dqt[0] * a.scale, dqt[1] * a.scale),
                                 pack_bf16x2(dqt[2] * a.scale, dqt[3] * a.scale)});
          } else {
            const float4 x{dqt[0] * a.scale, dqt[1] * a.scale, dqt[2] * a.scale, dqt[3] * a.scale};
            store16_nt(dst, &x);
          }
        }
      }
    }
    __syncthreads();  // the next round restages s_q, s_do, s_p, s_ds
  }
  // this chunk's share of dK, dV: lane (g, col) holds dims db*16 + 4g + i of key kb*16 + col
#pragma unroll
  for (int di = 0; di < DBW; ++di) {
    const int db = w * DBW + di;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int key = kb * 16 + col;
      if (key < nkeys) {
        float* dkr = a.dk_acc + (bh * a.N + key0 + key) * D + db * 16 + 4 * g;
        float* dvr = a.dv_acc + (bh * a.N + key0 + key) * D + db * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          atomicAdd(dkr + i, dkt[di][kb][i] * a.scale);
          atomicAdd(dvr + i, dvt[di][kb][i]);
        }
      }
    }
  }
}

// ---- dq = sum of the K partial rows of every (query, head) -----------------------
struct BwdMergeArgs {
  const int32_t* idx;
  const void* dq_part;  // input dtype
  void* dq;
  int64_t head0, heads, M1;
  int32_t N, Hq, Hkv, K;
};

// One wave per (query, KV head): the valid slots as a lane mask, then each
// lane (8 dims of one head) issues the loads of up to 16 slots' rows at once
// and sums them.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void bwd_merge_kernel(BwdMergeArgs a) {
  constexpr int SG = 16;
  const int64_t wid = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (wid >= a.heads * a.N) return;
  const int lane = lane_id();
  const int64_t hl = wid / a.N, t = wid % a.N;
  const int64_t bh = a.head0 + hl;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int32_t* sel = a.idx + (bh * a.N + t) * a.K;
  const int64_t rec0 = (hl * a.N + t) * a.K * G;
  const int32_t js = lane < a.K ? sel[lane] : -1;
  const uint64_t okm = __ballot(js >= 0 && js < a.M1);  // K <= 32
  const T* part = static_cast<const T*>(a.dq_part);
  for (int e0 = lane * 8; e0 < G * D; e0 += kWave * 8) {
    const int hh = e0 / D, d = e0 % D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.K; s0 += SG) {
      Row8<T> rows[SG];
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        const int s = s0 + u;
        if (s < a.K && ((okm >> s) & 1ull)) rows[u].load_nt(part + (rec0 + s * G + hh) * D + d);
        else rows[u] = Row8<T>{};
      }
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        float v[8];
        rows[u].get(v);  // zero for an invalid slot
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
    T* out = static_cast<T*>(a.dq) + (((int64_t)b * a.Hq + h * G + hh) * a.N + t) * D + d;
#pragma unroll
    for (int i = 0; i < 8; ++i) store1<T>(out + i, acc[i]);
  }
}

__global__ void zero_f32_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// dk, dv [B][Hkv][cap][D] rows < N from the fp32 accumulators [B][Hkv][N][D]
template <typename T>
__global__ void bwd_store_kernel(const float* __restrict__ acc, T* out, int64_t BH, int64_t N, int64_t cap,
                                 int32_t D) {
  const int64_t n = BH * N * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / D, d = i % D;
    const int64_t bh = row / N, r = row % N;
    store1<T>(out + (bh * cap + r) * D + d, acc[i]);
  }
}

hipError_t launch_attn_bwd(const Problem& p, const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           hipStream_t stream) {
  const BwdLayout L = bwd_layout(p);
  char* base = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.off_counts);
  int32_t* cursor = reinterpret_cast<int32_t*>(base + L.off_cursor);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.off_offsets);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + L.off_chunks);
  ChunkEntry* chunk_map = reinterpret_cast<ChunkEntry*>(base + L.off_map);
  int32_t* pairs = reinterpret_cast<int32_t*>(base + L.off_pairs);
  void* dq_part = base + L.off_dq;
  float* rowdot = reinterpret_cast<float*>(base + L.off_rowdot);
  float* dk_acc = reinterpret_cast<float*>(base + L.off_dk);
  float* dv_acc = reinterpret_cast<float*>(base + L.off_dv);
  const int64_t BH = (int64_t)p.B * p.Hkv;
  const int64_t acc_n = BH * p.N * p.D;
  const unsigned zb = (unsigned)((acc_n + 255) / 256 < 65536 ? (acc_n + 255) / 256 : 65536);
  PISA_LAUNCH("bwd_zero", stream, zero_f32_kernel, dim3(zb), dim3(256), 0, dk_acc, acc_n);
  PISA_LAUNCH("bwd_zero", stream, zero_f32_kernel, dim3(zb), dim3(256), 0, dv_acc, acc_n);
  hipError_t err = dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    const int64_t rows = (int64_t)p.B * p.Hq * p.N;
    const int64_t threads = rows * (D / 8);
    PISA_LAUNCH("bwd_rowdot", stream, (rowdot_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                static_cast<const T*>(dout), static_cast<const T*>(o), rows, rowdot);
    return hipGetLastError();
  });
  if (err != hipSuccess) return err;
  for (int64_t head0 = 0; head0 < BH; head0 += L.heads) {
    const int64_t heads = (BH - head0) < L.heads ? (BH - head0) : L.heads;
    const int64_t entries = heads * p.N * p.K;
    const int64_t ncl = heads * L.Mb;
    const ClusterBufs cb{counts, cursor, offsets, chunk_off, pairs, reinterpret_cast<int32_t*>(base + L.off_hist)};
    err = launch_clusters(idx + head0 * p.N * p.K, heads, (int64_t)p.N * p.K, p.K, L.M1, kAttnBins, bwd_chunk(p), cb, stream);
    if (err != hipSuccess) return err;
    const int64_t max_chunks = (entries + bwd_chunk(p) - 1) / bwd_chunk(p) + ncl;
    err = launch_chunk_map(chunk_off, offsets, counts, ncl, bwd_chunk(p), max_chunks, chunk_map, stream);
    if (err != hipSuccess) return err;
    BwdArgs ba{q, k, v, dout, lse, rowdot, counts, offsets, chunk_off, chunk_map, pairs, dq_part, dk_acc, dv_acc, ncl, L.M1, L.Mb,
               head0, p.N, p.Hq, p.Hkv, p.C, p.K, bwd_chunk(p), p.causal ? 1 : 0, p.cap, p.scale};
    BwdMergeArgs ma{idx, dq_part, dq, head0, heads, L.M1, p.N, p.Hq, p.Hkv, p.K};
    err = dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
      using T = std::remove_pointer_t<decltype(tp)>;
      constexpr int D = decltype(dc)::value;
      constexpr int G = decltype(gc)::value;
      auto run = [&](auto kern, int nkb, int nw) -> hipError_t {
        const int cp = nkb * 16, epv = 16 / (int)sizeof(T);
        const size_t lds = (2 * (size_t)cp * (D + epv) + (size_t)D * (cp + epv)) * sizeof(T);
        if (lds > 65536) {
          hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (e != hipSuccess) return e;
        }
        PISA_LAUNCH("attn_bwd", stream, kern, dim3((unsigned)max_chunks), dim3(nw * kWave), lds, ba);
        return hipGetLastError();
      };
      hipError_t e;
      if (p.C <= 32)
        e = run(attn_bwd_kernel<T, D, G, 2>, 2, bwd_waves<D, 2>());
      else if (p.C <= 64)
        e = run(attn_bwd_kernel<T, D, G, 4>, 4, bwd_waves<D, 4>());
      else
        e = run(attn_bwd_kernel<T, D, G, 8>, 8, bwd_waves<D, 8>());
      if (e != hipSuccess) return e;
      const int64_t waves = heads * p.N;
      PISA_LAUNCH("bwd_merge", stream, (bwd_merge_kernel<T, D, G>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                  ma);
      return hipGetLastError();
    });
    if (err != hipSuccess) return err;
  }
  return dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto, auto) -> hipError_t {
    using T = std::remove_pointer_t<decltype(tp)>;
    PISA_LAUNCH("bwd_store", stream, bwd_store_kernel<T>, dim3(zb), dim3(256), 0, dk_acc, static_cast<T*>(dk), BH,
                (int64_t)p.N, p.cap, p.D);
    PISA_LAUNCH("bwd_store", stream, bwd_store_kernel<T>, dim3(zb), dim3(256), 0, dv_acc, static_cast<T*>(dv), BH,
                (int64_t)p.N, p.cap, p.D);
    return hipGetLastError();
  });
}

}  // namespace pisa
