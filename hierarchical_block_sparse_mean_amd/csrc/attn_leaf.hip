// Leaf-major block-sparse attention on MFMA ("Block Sparse Attention with
// Log-Linear Complexity", hyper.ai page, section "block-sparse attention",
// the o_t equation: softmax over the raw keys of the kept blocks, applied to
// their raw values).
//
// The kept (query, leaf) pairs are grouped by (query block, leaf) (the same
// histogram / scan / scatter as the selector's clusters).  One workgroup
// holds a leaf's C keys (row-major) and values (transposed) in LDS and
// streams the queries of the block that kept it, 16 MFMA columns = 16 / G_Q
// queries x G_Q heads at a time, the next tile's query rows in flight:
//   S^T = K Q^T        (C x 16, v_mfma_f32_16x16x32_bf16, fp32 accumulate)
//   P^T = exp(S^T - m) per column (the accumulator layout already is the
//                      B-operand layout of the next product: no LDS trip)
//   O^T = V^T P^T      (d x 16)
// and writes a partial (m, l, O) per (query, slot, head).  A merge pass per
// (query, KV head) combines the K partials into o and lse.  Partial O is
// stored in the input dtype (bf16 rounding is far inside the bf16 tolerance).
// The partial records are written and read with streaming (nontemporal)
// stores and loads: each is touched once on each side, and left to the
// normal policy they displace the query rows and key tiles the leaf kernel
// reuses (128K attention 6.7 -> 5.7 ms).
// Where a query kept both leaves of a level-2 block (2j and 2j + 1, adjacent
// in its ascending row) and 2C keys fit one tile (C <= 64, or C <= 128 for
// 16-bit inputs, whose 256-key tile leaves LDS for five waves), the pair goes
// to a cluster of that block instead: a second launch attends the 2C keys in
// one tile, so the query's rows are read once and one partial (under the slot
// of the even leaf) is written for both; the merge recognises the odd leaf's
// slot from idx and skips it.
// Work is done in chunks of KV heads so that the partial buffers stay within
// a bound (24 GiB: all eight KV heads at once at 128K, two at a time at 256K).
#include "kernels.h"

namespace pisa {

// (query, slot) pairs per workgroup, at most: 512 for leaves of C <= 64 keys,
// 1024 for longer ones (a longer chunk re-stages a leaf's K and V fewer
// times; measured best per leaf size)
constexpr int kAttnChunk = 1024;
static int attn_chunk(const Problem& p) { return p.C > 64 ? 1024 : 512; }
constexpr size_t kLdsPerCu = 160 * 1024;
// Tiles of this many 16-key blocks or more (the 256-key sibling-pair tiles
// of 16-bit inputs at C = 128) store their partial rows straight from the
// accumulators: the LDS the output staging would take is what limited them
// to five waves per CU; without it eight fit (256K attention 32.2 -> 27.7 ms).
// Smaller tiles stage through LDS and store whole rows, which measured
// faster for them (128K: 5.5 vs 7.2 ms with register stores everywhere).
constexpr int kAttnRegStoreNKB = 16;

// V^T row pad (elements): rows 4 elements apart in bank offset, so the 8-byte
// reads of 16 consecutive dims (rows) at one key offset fall in distinct
// banks whether a pass serves 32 or 64 banks
constexpr int kVtPad = 4;

// LDS of a workgroup: the tile's K (row-major) and V^T, the waves' output
// staging, the chunk's pair codes
template <typename T, int D, int NKB>
constexpr size_t attn_lds_bytes(int nw) {
  constexpr size_t e = 16 / sizeof(T);
  const size_t staging = (size_t)(NKB >= kAttnRegStoreNKB ? 1 : nw) * 16 * (D + e);
  return ((size_t)NKB * 16 * (D + e) + (size_t)D * (NKB * 16 + kVtPad) + staging) * sizeof(T) + 4 * (size_t)kAttnChunk;
}
// waves per workgroup: 12 for tiles of 8 key blocks (their K, V^T and the
// waves' output staging leave room for one workgroup per CU, so it brings
// the waves), 8 for 16-block tiles (no output staging; their registers allow
// two waves per SIMD) and for smaller tiles (two workgroups per CU); fewer
// where that would not fit the LDS (fp32 rows of d = 128 in 8-block tiles)
template <typename T, int D, int NKB>
constexpr int attn_waves() {
  int nw = NKB >= 16 ? 8 : (NKB >= 8 ? 12 : 8);
  while (nw > 1 && attn_lds_bytes<T, D, NKB>(nw) > kLdsPerCu) --nw;
  return nw;
}
constexpr size_t kAttnBudget = (size_t)24 << 30;  // partial buffers per head chunk

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// sibling pairing: level-2 block tiles of 2C keys, at most 8 key blocks, or
// 16 for 16-bit inputs (five waves fit beside a 256-key tile: 256K attention
// 47.9 -> 46.4 ms, the merge reading fewer partials); not for fp32 rows of
// d = 128 (an 8-block tile leaves LDS for two waves only), nor
// where the level-2 blocks would push a head's clustering off its LDS
// histogram (M_1 <= 16384 < M_1 + M_2: from about 700K to 1M tokens at
// C = 64; measured 95 ms unpaired against 105 ms paired at 1M).  Beyond, both
// take the global-atomic path and pairing pays again.
static bool attn_pairs(const Problem& p) {
  const int64_t M1 = level_rows(p.N, p.C, 1);
  const bool leaves_in_lds = M1 <= kClusterLdsBins;
  const bool pairs_in_lds = M1 + (M1 + 1) / 2 <= kClusterLdsBins;
  return (p.C <= 64 ? (p.dtype == 1 || p.D <= 64) : p.dtype == 1) && (pairs_in_lds || !leaves_in_lds);
}

struct AttnLayout {
  int64_t heads;  // (b, h) heads per chunk
  int64_t M1, Mk, Mb, ncl, slots, max_chunks;  // Mk: key blocks (leaves, then level-2 blocks); Mb: bins per head
  size_t off_counts, off_cursor, off_offsets, off_chunks, off_map, off_pairs, off_ml, off_o, off_hist, total;
};

static AttnLayout attn_layout(const Problem& p) {
  AttnLayout L{};
  const size_t osz = p.dtype == 1 ? 2 : 4;
  L.M1 = level_rows(p.N, p.C, 1);
  L.Mk = L.M1 + (attn_pairs(p) ? (L.M1 + 1) / 2 : 0);
  L.Mb = cluster_bins(p.N, L.Mk, kAttnBins);
  const size_t per_head = (size_t)p.N * p.K * (4 + (size_t)p.G * (8 + p.D * osz)) + (size_t)L.Mb * 20 +
                          (size_t)p.N * p.K / attn_chunk(p) * 4;
  const int64_t BH = (int64_t)p.B * p.Hkv;
  int64_t hmax = (int64_t)(kAttnBudget / per_head);
  if (hmax < 1) hmax = 1;
  if (hmax > BH) hmax = BH;
  const int64_t nchunks = (BH + hmax - 1) / hmax;
  L.heads = (BH + nchunks - 1) / nchunks;
  L.ncl = L.heads * L.Mb;
  L.slots = L.heads * (int64_t)p.N * p.K;
  L.max_chunks = (L.slots + attn_chunk(p) - 1) / attn_chunk(p) + L.ncl;
  size_t off = 0;
  L.off_counts = off;
  off = a256(off + 4 * (size_t)L.ncl);
  L.off_cursor = off;
  off = a256(off + 4 * (size_t)L.ncl);
  L.off_offsets = off;
  off = a256(off + 4 * (size_t)(L.ncl + 1));
  L.off_chunks = off;
  off = a256(off + 4 * (size_t)(L.ncl + 1));
  L.off_map = off;
  off = a256(off + sizeof(ChunkEntry) * (size_t)L.max_chunks);
  L.off_pairs = off;
  off = a256(off + 4 * (size_t)L.slots);
  L.off_ml = off;
  off = a256(off + 8 * (size_t)L.slots * p.G);
  L.off_o = off;
  off = a256(off + osz * (size_t)L.slots * p.G * p.D);
  L.off_hist = off;
  off = a256(off + cluster_scratch_bytes(L.heads, (int64_t)p.N * p.K, L.Mb));
  L.total = off;
  return L;
}

size_t attn_leaf_workspace_bytes(const Problem& p) { return attn_layout(p).total; }

struct AttnLeafArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* chunk_off;
  const ChunkEntry* chunk_map;  // work chunk -> (cluster, first pair, pairs)
  const int32_t* pairs;
  floatx2_t* pml;  // (m, l) [heads][N][K][G]
  void* po;    // [heads][N][K][G][D] (input dtype)
  int64_t ncl, M1, Mk, Mb, head0;
  int32_t N, Hq, Hkv, C, K;
  int32_t chunk;  // pairs per work chunk (<= kAttnChunk)
  int32_t causal;
  int64_t cap;
  float scale;
};

// NKB: 16-key blocks covering the tile (even, Ct <= 16 NKB), Ct = C keys of
// a leaf, or 2C of a level-2 block (PAIRED: the launch over the level-2
// block clusters; each launch skips the other kind's chunks).
template <typename T, int D, int G, int NKB, bool PAIRED>
__global__ __launch_bounds__((attn_waves<T, D, NKB>() * kWave)) PISA_MFMA_REGS void attn_leaf_kernel(AttnLeafArgs a) {
  constexpr int NW = attn_waves<T, D, NKB>();
  constexpr int NS = D / 32;                   // contraction steps of S
  constexpr int TQ = 16 / G;                   // queries per 16-column tile
  constexpr int CP = NKB * 16;                 // keys held (zero padded)
  constexpr int KP = D + 16 / (int)sizeof(T);  // K row pitch
  constexpr int VP = CP + kVtPad;              // V^T row pitch
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* s_k = reinterpret_cast<T*>(smem_raw);  // [CP][KP]
  T* s_vt = s_k + CP * KP;                   // [D][VP]
  // a tile's 16 output columns x D, staged so each lane stores 16-byte pieces
  // (tiles that store from registers keep a one-wave placeholder)
  __shared__ __align__(16) T s_o[NKB >= kAttnRegStoreNKB ? 1 : NW][16][D + 16 / sizeof(T)];
  __shared__ int32_t s_pr[kAttnChunk];  // the chunk's pair codes

  const ChunkEntry ce = a.chunk_map[blockIdx.x];
  if (ce.cluster < 0) return;  // past the last work chunk (uniform over the workgroup)
  const int64_t c = ce.cluster;
  const int64_t hl = c / a.Mb;  // head within the chunk
  const int64_t jk = c % a.Mk;  // key block: leaf, or M_1 + level-2 block
  if ((jk >= a.M1) != PAIRED) return;  // the other launch's cluster
  const int64_t bh = a.head0 + hl;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int64_t p_begin = ce.begin;
  const int64_t p_end = p_begin + ce.count;

  const int C = PAIRED ? 2 * a.C : a.C;  // keys of the tile
  const int64_t key0 = (PAIRED ? jk - a.M1 : jk) * (int64_t)C;
  const int nkeys = (int)((a.N - key0) < C ? (a.N - key0) : C);
  const T* kh = static_cast<const T*>(a.k) + bh * a.cap * D;
  const T* vh = static_cast<const T*>(a.v) + bh * a.cap * D;
  constexpr int EPV = 16 / sizeof(T);
  for (int i = threadIdx.x; i < CP * (D / EPV); i += blockDim.x) {
    const int r = i / (D / EPV), d = (i % (D / EPV)) * EPV;
    uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (r < nkeys) {
      kv = *reinterpret_cast<const uint4*>(kh + (key0 + r) * D + d);
      vv = *reinterpret_cast<const uint4*>(vh + (key0 + r) * D + d);
    }
    *reinterpret_cast<uint4*>(s_k + r * KP + d) = kv;
    const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int e = 0; e < EPV; ++e) s_vt[(d + e) * VP + r] = ve[e];
  }
  for (int i = threadIdx.x; i < a.chunk; i += blockDim.x)
    s_pr[i] = p_begin + i < p_end ? a.pairs[p_begin + i] : -1;
  __syncthreads();

  const int w = threadIdx.x / kWave, lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const int qi = col / G, hh = col % G;
  const T* qb = static_cast<const T*>(a.q);
  // column col of a tile = query qi (its pair) x head hh; the B operand of
  // S^T = K Q^T is that query head's row.  An empty column (pr < 0) reads
  // query 0's row (finite data, never stored).
  auto load_q = [&](int32_t pr, Frag<T>* f) {
    const int64_t tq = pr >= 0 ? (pr >> 5) : 0;
    const T* qrow = qb + (((int64_t)b * a.Hq + h * G + hh) * a.N + tq) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) f[s].load(qrow + 32 * s + 8 * g);
  };
  // one tile of 16 / G_Q pairs; MASK: some column of the chunk sees fewer
  // keys than the tile holds (causal diagonal leaf, last leaf, zero padding)
  auto attend_tile = [&](const Frag<T>* fq, int32_t pr, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const bool live = pr >= 0;
    const int64_t t = live ? (pr >> 5) : -1;
    // K / V^T fragments are re-read from LDS every tile (an offset opaque to
    // the compiler keeps them from being held in registers across tiles)
    int toff = 0;
    asm volatile("" : "+v"(toff));
    const T* sk = s_k + toff;
    const T* svt = s_vt + toff;
    floatx4 acc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      acc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Frag<T> fk;
        fk.load(sk + (kb * 16 + col) * KP + 32 * s + 8 * g);
        acc[kb] = mma(fk, fq[s], acc[kb]);
      }
    }
    // column softmax statistics (keys are rows 4g+i of each 16-key block):
    // max on the raw dot products, then p = exp2((x - max) * scale*log2e)
    if constexpr (MASK) {
      const int lim = live ? (int)(a.causal ? (t - key0 + 1 < nkeys ? t - key0 + 1 : nkeys) : nkeys) : 0;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kb][i] = kb * 16 + 4 * g + i >= lim ? -INFINITY : acc[kb][i];
    }
    float mraw = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mraw = fmaxf(mraw, acc[kb][i]);
    mraw = rows_max(mraw);
    const float sl2 = a.scale * 1.4426950408889634f;
    const float nb = -mraw * sl2;
    float l = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2_nonpos(fmaf(acc[kb][i], sl2, nb));  // exp2(-inf) = 0
        acc[kb][i] = pv;
        l += pv;
      }
    l = rows_sum(l);
    const float m = mraw * a.scale;  // the partial's max logit (natural units)
    // O^T = V^T P^T, contraction over 32 keys = 16-key blocks (2s, 2s+1)
    floatx4 oacc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < NKB / 2; ++sp) {
      const float pk[8] = {acc[2 * sp][0],     acc[2 * sp][1],     acc[2 * sp][2],     acc[2 * sp][3],
                           acc[2 * sp + 1][0], acc[2 * sp + 1][1], acc[2 * sp + 1][2], acc[2 * sp + 1][3]};
      Frag<T> fp;
      fp.set(pk);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        Frag<T> fv;
        const T* row = svt + (db * 16 + col) * VP;
        fv.load4x2(row + (2 * sp) * 16 + 4 * g, row + (2 * sp + 1) * 16 + 4 * g);
        oacc[db] = mma(fv, fp, oacc[db]);
      }
    }
    if constexpr (NKB >= kAttnRegStoreNKB) {
      // lane (col, g) holds dims 16 db + 4g + [0, 4) of column col; a row
      // swap between lane groups g and g ^ 1 (v_permlane16_swap) turns each
      // pair of d-blocks (2p, 2p + 1) into 8 consecutive dims per lane
      // (group 0: [32p, +8), 1: [32p + 16, +8), 2: [32p + 8, +8),
      // 3: [32p + 24, +8)), so a column's four lanes store 64 contiguous
      // bytes per instruction; fp32 rows already hold 16 contiguous bytes
      if (live) {
        const int64_t rec = ((hl * a.N + t) * a.K + (pr & 31)) * G + hh;
        T* dst = static_cast<T*>(a.po) + rec * D;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int pp = 0; pp < D / 32; ++pp) {
            const uint32_t a0 = pack_bf16x2(oacc[2 * pp][0], oacc[2 * pp][1]);
            const uint32_t a1 = pack_bf16x2(oacc[2 * pp][2], oacc[2 * pp][3]);
            const uint32_t b0 = pack_bf16x2(oacc[2 * pp + 1][0], oacc[2 * pp + 1][1]);
            const uint32_t b1 = pack_bf16x2(oacc[2 * pp + 1][2], oacc[2 * pp + 1][3]);
            const auto r0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
            const auto r1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
            const uint4 x{r0[0], r1[0], r0[1], r1[1]};
            store16_nt(dst + 32 * pp + (g & 1) * 16 + (g >> 1) * 8, &x);
          }
        } else {
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            const float4 x{oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]};
            store16_nt(dst + db * 16 + 4 * g, &x);
          }
        }
        if (g == 0) __builtin_nontemporal_store(floatx2_t{m, l}, a.pml + rec);  // one 8-byte store per record
      }
    } else {
      // partial record of (query, slot, head): column col holds rows 4g+i of
      // each d-block; stage the 16 x D tile in LDS, then store whole rows
      // (the lane's 4 dims of a d-block are consecutive: one 8- or 16-byte store)
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        T* dst = &s_o[w][col][db * 16 + 4 * g];
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(oacc[db][0], oacc[db][1]), pack_bf16x2(oacc[db][2], oacc[db][3])};
        else
          *reinterpret_cast<float4*>(dst) = float4{oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]};
      }
      if (live && g == 0) {
        const int64_t rec = ((hl * a.N + t) * a.K + (pr & 31)) * G + hh;
        __builtin_nontemporal_store(floatx2_t{m, l}, a.pml + rec);  // one 8-byte store per (query, slot, head)
      }
      wave_sync();
      {
        constexpr int CH = 16 / (int)sizeof(T);  // elements per 16-byte piece
        constexpr int PER_COL = D / CH;
#pragma unroll
        for (int it = 0; it < 16 * PER_COL / kWave; ++it) {
          const int i = it * kWave + lane;
          const int cc = i / PER_COL, piece = i % PER_COL;
          const int32_t pc = __shfl(pr, cc);  // pair of column cc (lane cc of group 0)
          if (pc >= 0) {
            const int64_t rec = ((hl * a.N + (pc >> 5)) * a.K + (pc & 31)) * G + (cc % G);
            store16_nt(static_cast<T*>(a.po) + rec * D + piece * CH, &s_o[w][cc][piece * CH]);
          }
        }
      }
      wave_sync();
    }
  };
  // tiles w, w + W, ... of the chunk (W = waves), two query-row buffers: the
  // next tile's rows load while the current tile is attended
  const int n = (int)(p_end - p_begin);
  const int stride = NW * TQ;
  auto pair_at = [&](int i) -> int32_t { return i + qi < n ? s_pr[i + qi] : -1; };
  auto run = [&](auto mask_c) {
    Frag<T> fa[NS], fb[NS];
    int i = w * TQ;
    if (i >= n) return;
    int32_t pa = pair_at(i), pb;
    load_q(pa, fa);
    while (true) {
      pb = pair_at(i + stride);
      load_q(pb, fb);
      attend_tile(fa, pa, mask_c);
      i += stride;
      if (i >= n) break;
      pa = pair_at(i + stride);
      load_q(pa, fa);
      attend_tile(fb, pb, mask_c);
      i += stride;
      if (i >= n) break;
    }
  };
  // zero-padded keys (C < 16 NKB) always need the mask; otherwise only chunks
  // holding a query that sees fewer than C keys of the leaf
  bool part = CP > C;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t tq = s_pr[i] >> 5;
    part |= (a.causal && tq - key0 + 1 < C) || nkeys < C;
  }
  if (__syncthreads_or(part)) run(std::true_type{});
  else run(std::false_type{});
}

// ---- merge the K partials of every (query, KV head) ---------------------------
struct MergeArgs {
  const int32_t* idx;
  const floatx2_t* pml;
  const void* po;
  void* o;
  float* lse;
  int64_t head0, heads, M1;
  int32_t N, Hq, Hkv, K;
  int32_t pairs;  // sibling pairs were attended as one partial (under the even leaf's slot)
};

// One wave per (query, KV head).  The slots that hold a partial follow from
// idx alone (a leaf of the problem, other than the odd half of a kept
// sibling pair when pairs were attended together), so each lane, which owns
// 8 output dims of one head, issues the loads of its first SG slots' rows
// before the slots' m and l (staged through LDS) have arrived; the rows are
// then combined with weights exp(m - max m).  SG: slots whose rows are loaded
// together (K rounded up to 16 or 32 for 16-bit rows, half that for fp32).
template <typename T, int D, int G, int SG>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int MLP = (32 * G + kWave - 1) / kWave;   // (m, l) entries per lane, at most
  __shared__ float s_m[4][32 * G], s_l[4][32 * G];
  __shared__ int32_t s_ok[4][32];
  const int w = threadIdx.x / kWave;
  const int64_t wid = (int64_t)blockIdx.x * 4 + w;
  if (wid >= a.heads * a.N) return;
  const int lane = lane_id();
  const int64_t hl = wid / a.N, t = wid % a.N;
  const int64_t bh = a.head0 + hl;
  const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
  const int32_t* sel = a.idx + (bh * a.N + t) * a.K;
  const int64_t rec0 = (hl * a.N + t) * a.K * G;  // record of (slot 0, head 0)
  for (int i = lane; i < a.K; i += kWave) {
    const int32_t j = sel[i];
    bool ok = j >= 0 && j < a.M1;
    if (ok && a.pairs && (j & 1) && i > 0 && sel[i - 1] == j - 1) ok = false;
    s_ok[w][i] = ok ? 1 : 0;
  }
  float mv[MLP], lv[MLP];
#pragma unroll
  for (int r = 0; r < MLP; ++r) {
    const int i = lane + r * kWave;
    const floatx2_t ml = i < a.K * G ? __builtin_nontemporal_load(a.pml + rec0 + i) : floatx2_t{0.f, 0.f};
    mv[r] = ml[0];
    lv[r] = ml[1];
  }
  wave_sync();  // s_ok
  const T* po = static_cast<const T*>(a.po);
  auto issue = [&](int e0, int s0, Row8<T>* rows) {
    const int hh = e0 / D, d = e0 % D;
#pragma unroll
    for (int u = 0; u < SG; ++u) {
      const int s = s0 + u;
      if (s < a.K && s_ok[w][s]) rows[u].load_nt(po + (rec0 + s * G + hh) * D + d);
      else rows[u] = Row8<T>{};
    }
  };
  // where one pass of the lanes covers the G heads (G d <= 512), the first
  // SG rows are in flight while m and l are staged
  constexpr bool ONE = G * D <= 8 * kWave;
  const int e_first = lane * 8;
  Row8<T> first[ONE ? SG : 1];
  if constexpr (ONE)
    if (e_first < G * D) issue(e_first, 0, first);
#pragma unroll
  for (int r = 0; r < MLP; ++r) {
    const int i = lane + r * kWave;
    if (i < a.K * G) {
      s_m[w][i] = mv[r];
      s_l[w][i] = lv[r];
    }
  }
  wave_sync();  // s_m, s_l
  for (int e0 = e_first; e0 < G * D; e0 += kWave * 8) {
    const int hh = e0 / D, d = e0 % D;
    float M = -INFINITY;
    for (int s = 0; s < a.K; ++s)
      if (s_ok[w][s]) M = fmaxf(M, s_m[w][s * G + hh]);
    float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const Row8<T>* rows, int s0) {
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        const int s = s0 + u;
        if (s < a.K && s_ok[w][s] && s_m[w][s * G + hh] != -INFINITY) {
          const float wgt = __expf(s_m[w][s * G + hh] - M);
          L += wgt * s_l[w][s * G + hh];
          float v[8];
          rows[u].get(v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wgt, v[i], acc[i]);
        }
      }
    };
    if (M != -INFINITY) {
      int s0 = 0;
      if constexpr (ONE) {
        consume(first, 0);
        s0 = SG;
      }
      for (; s0 < a.K; s0 += SG) {
        Row8<T> rows[SG];
        issue(e0, s0, rows);
        consume(rows, s0);
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* out = static_cast<T*>(a.o) + (((int64_t)b * a.Hq + h * G + hh) * a.N + t) * D + d;
    if constexpr (sizeof(T) == 2) {
      uint32_t wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wv[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
      const uint4 x{wv[0], wv[1], wv[2], wv[3]};
      store16_nt(out, &x);  // o is not read again here
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) store1<T>(out + i, acc[i] * inv);
    }
    if (a.lse != nullptr && d == 0)
      a.lse[((int64_t)b * a.Hq + h * G + hh) * a.N + t] = L > 0.f ? M + __logf(L) : -INFINITY;
  }
}

hipError_t launch_attn_leaf(const Problem& p, const void* q, const void* k, const void* v, const int32_t* idx,
                            void* o, float* lse, void* ws, hipStream_t stream) {
  const AttnLayout L = attn_layout(p);
  const bool pairs_on = attn_pairs(p);
  char* base = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.off_counts);
  int32_t* cursor = reinterpret_cast<int32_t*>(base + L.off_cursor);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.off_offsets);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + L.off_chunks);
  ChunkEntry* chunk_map = reinterpret_cast<ChunkEntry*>(base + L.off_map);
  int32_t* pairs = reinterpret_cast<int32_t*>(base + L.off_pairs);
  floatx2_t* pml = reinterpret_cast<floatx2_t*>(base + L.off_ml);
  void* po = base + L.off_o;
  const int64_t BH = (int64_t)p.B * p.Hkv;
  for (int64_t head0 = 0; head0 < BH; head0 += L.heads) {
    const int64_t heads = (BH - head0) < L.heads ? (BH - head0) : L.heads;
    const int64_t entries = heads * p.N * p.K;
    const int64_t ncl = heads * L.Mb;
    const ClusterBufs cb{counts, cursor, offsets, chunk_off, pairs, reinterpret_cast<int32_t*>(base + L.off_hist)};
    hipError_t err = launch_clusters(idx + head0 * p.N * p.K, heads, (int64_t)p.N * p.K, p.K, L.Mk, kAttnBins,
                                     attn_chunk(p), cb, stream, pairs_on ? L.M1 : 0);
    if (err != hipSuccess) return err;
    const int64_t max_chunks = (entries + attn_chunk(p) - 1) / attn_chunk(p) + ncl;
    err = launch_chunk_map(chunk_off, offsets, counts, ncl, attn_chunk(p), max_chunks, chunk_map, stream);
    if (err != hipSuccess) return err;
    AttnLeafArgs aa{q, k, v, counts, offsets, chunk_off, chunk_map, pairs, pml, po, ncl, L.M1, L.Mk, L.Mb, head0,
                    p.N, p.Hq, p.Hkv, p.C, p.K, attn_chunk(p), p.causal ? 1 : 0, p.cap, p.scale};
    MergeArgs ma{idx, pml, po, o, lse, head0, heads, L.M1, p.N, p.Hq, p.Hkv, p.K, pairs_on ? 1 : 0};
    err = dispatch_tdg(p.dtype, p.D, p.G, [&](auto tp, auto dc, auto gc) -> hipError_t {
      using T = std::remove_pointer_t<decltype(tp)>;
      constexpr int D = decltype(dc)::value;
      constexpr int G = decltype(gc)::value;
      auto run = [&](auto kern, int nkb, int nw) -> hipError_t {
        const size_t lds = ((size_t)nkb * 16 * (D + 16 / sizeof(T)) + (size_t)D * (nkb * 16 + kVtPad)) *
                           sizeof(T);
        if (lds > 65536) {
          hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          if (e != hipSuccess) return e;
        }
        PISA_LAUNCH("attn_leaf", stream, kern, dim3((unsigned)max_chunks), dim3(nw * kWave), lds, aa);
        return hipGetLastError();
      };
      hipError_t e;
      if (p.C <= 32) {
        e = run(attn_leaf_kernel<T, D, G, 2, false>, 2, attn_waves<T, D, 2>());
        if (e == hipSuccess && pairs_on) e = run(attn_leaf_kernel<T, D, G, 4, true>, 4, attn_waves<T, D, 4>());
      } else if (p.C <= 64) {
        e = run(attn_leaf_kernel<T, D, G, 4, false>, 4, attn_waves<T, D, 4>());
        if (e == hipSuccess && pairs_on) e = run(attn_leaf_kernel<T, D, G, 8, true>, 8, attn_waves<T, D, 8>());
      } else {
        e = run(attn_leaf_kernel<T, D, G, 8, false>, 8, attn_waves<T, D, 8>());
        if constexpr (sizeof(T) == 2)
          if (e == hipSuccess && pairs_on) e = run(attn_leaf_kernel<T, D, G, 16, true>, 16, attn_waves<T, D, 16>());
      }
      if (e != hipSuccess) return e;
      const int64_t waves = heads * p.N;
      const dim3 mgrid((unsigned)((waves + 3) / 4));
      constexpr int sg = sizeof(T) == 2 ? 16 : 8;
      if (p.K <= sg)
        PISA_LAUNCH("attn_merge", stream, (attn_merge_kernel<T, D, G, sg>), mgrid, dim3(256), 0, ma);
      else
        PISA_LAUNCH("attn_merge", stream, (attn_merge_kernel<T, D, G, 2 * sg>), mgrid, dim3(256), 0, ma);
      return hipGetLastError();
    });
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace pisa
