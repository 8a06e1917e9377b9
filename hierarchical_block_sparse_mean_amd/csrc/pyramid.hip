// Mean-pooled key pyramid ("Block Sparse Attention with Log-Linear
// Complexity", hyper.ai page, section "pyramid key-block hierarchy": level 0 =
// raw keys, the first merge uses g_0 = C and yields the leaves, every higher
// merge uses g = 2, M_{l+1} = ceil(M_l / g_l), and each summary is the mean of
// its children's summaries).
//
// pyr_leaf_kernel: one workgroup per (b, h, chunk of 16 leaves); coalesced
// 16-byte loads of the raw keys (one HBM pass), leaf means, then the four
// levels above the chunk from LDS.  pyr_up_kernel: one workgroup per
// (b, h, chunk of 64 blocks of a base level), six more levels from LDS.
#include "kernels.h"

namespace pisa {

constexpr int kLeafChunk = 16;  // leaves per workgroup (4 levels above them)
constexpr int kLeafLevels = 4;
constexpr int kUpChunk = 64;    // base blocks per workgroup (6 levels above)
constexpr int kUpLevels = 6;

struct PyrArgs {
  const void* k;
  float* pyr;
  _Float16* f16;  // block-floating-point copy: row * 2^-ex[row] in fp16
  int32_t* ex;    // per-row exponent (row index = element index / D)
  int64_t n;    // tokens
  int64_t cap;  // k row stride in tokens
  int32_t BH, C, L;
  PyrGeom geo;
};

// Builds levels lo+1 .. hi of the chunk from level lo held in buf (cnt0 rows,
// first global index first0) and writes them to global memory.
// fp16 block-floating-point copy of LDS rows [0, cnt) (global rows row0..),
// one wave per row.
template <int D>
__device__ __forceinline__ void put_f16_rows(const PyrArgs& a, const float* rows, int cnt, int64_t row0) {
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave, lane = lane_id();
  for (int p = w; p < cnt; p += nw) {
    float mx = 0.f;
    for (int d = lane; d < D; d += kWave) mx = fmaxf(mx, fabsf(rows[p * D + d]));
    const int e = row_exponent(wave_max(mx));
    for (int d = lane; d < D; d += kWave) a.f16[(row0 + p) * D + d] = to_f16_scaled(rows[p * D + d], e);
    if (lane == 0) a.ex[row0 + p] = e;
  }
}

template <int D>
__device__ __forceinline__ void build_levels_in_lds(float* buf0, float* buf1, int cnt0, int64_t first0,
                                                    int32_t lo, int32_t hi, const PyrArgs& a, int64_t head) {
  float* cur = buf0;
  float* nxt = buf1;
  int cnt = cnt0;
  int64_t first = first0;
  for (int32_t l = lo + 1; l <= hi; ++l) {
    const int64_t m_child = level_rows(a.n, a.C, l - 1);
    const int64_t m_par = level_rows(a.n, a.C, l);
    const int pcnt = (cnt + 1) / 2;
    const int64_t pfirst = first / 2;
    const int64_t dst = head + (a.geo.level_off[l] + pfirst) * D;
    const int pvalid = (int)((m_par - pfirst) < pcnt ? (m_par - pfirst) : pcnt);
    for (int i = threadIdx.x; i < pcnt * D; i += blockDim.x) {
      const int p = i / D, d = i % D;
      if (pfirst + p >= m_par) continue;
      const float c0 = cur[(2 * p) * D + d];
      const float v = (first + 2 * p + 1 < m_child) ? (c0 + cur[(2 * p + 1) * D + d]) * 0.5f : c0;
      nxt[p * D + d] = v;
      a.pyr[dst + p * D + d] = v;
    }
    __syncthreads();
    put_f16_rows<D>(a, nxt, pvalid, dst / D);
    float* tmp = cur;
    cur = nxt;
    nxt = tmp;
    cnt = pcnt;
    first = pfirst;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pyr_leaf_kernel(PyrArgs a) {
  constexpr int LPR = D / 8;           // lanes per key row (8 elements each)
  constexpr int RPP = kWave / LPR;     // rows per wave pass
  __shared__ float s_a[kLeafChunk * D];
  __shared__ float s_b[kLeafChunk / 2 * D];
  const int bh = (int)(blockIdx.x % a.BH);
  const int64_t chunk = blockIdx.x / a.BH;
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int rsub = lane / LPR, d0 = (lane % LPR) * 8;
  const T* kh = static_cast<const T*>(a.k) + (int64_t)bh * a.cap * D;
  const int64_t head = (int64_t)bh * a.geo.rows * D;
  const int64_t M1 = level_rows(a.n, a.C, 1);
  for (int li = w; li < kLeafChunk; li += 4) {
    const int64_t j = chunk * kLeafChunk + li;
    if (j >= M1) break;
    const int64_t lo = j * a.C;
    const int64_t cnt = (lo + a.C < a.n ? lo + a.C : a.n) - lo;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int64_t r = rsub; r < cnt; r += RPP) {
      float v[8];
      load8_nt<T>(kh + (lo + r) * D + d0, v);  // keys read once here (0.065 -> 0.058 ms at 128K)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = LPR; o < kWave; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
    if (lane < LPR) {
      const float cnt_f = (float)cnt;
      const int64_t dst = head + (a.geo.level_off[1] + j) * D + d0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float mval = acc[e] / cnt_f;
        s_a[li * D + d0 + e] = mval;
        a.pyr[dst + e] = mval;
      }
    }
  }
  __syncthreads();
  {
    const int64_t first = chunk * kLeafChunk;
    const int nleaf = (int)((M1 - first) < kLeafChunk ? (M1 - first) : kLeafChunk);
    put_f16_rows<D>(a, s_a, nleaf, (head + (a.geo.level_off[1] + first) * D) / D);
  }
  __syncthreads();
  const int64_t first = chunk * kLeafChunk;
  const int cnt0 = (int)((M1 - first) < kLeafChunk ? (M1 - first) : kLeafChunk);
  const int32_t hi = a.L < 1 + kLeafLevels ? a.L : 1 + kLeafLevels;
  build_levels_in_lds<D>(s_a, s_b, cnt0, first, 1, hi, a, head);
}

template <int D>
__global__ __launch_bounds__(256) void pyr_up_kernel(PyrArgs a, int32_t base_level) {
  __shared__ float s_a[kUpChunk * D];
  __shared__ float s_b[kUpChunk / 2 * D];
  const int bh = (int)(blockIdx.x % a.BH);
  const int64_t chunk = blockIdx.x / a.BH;
  const int64_t head = (int64_t)bh * a.geo.rows * D;
  const int64_t mb = level_rows(a.n, a.C, base_level);
  const int64_t first = chunk * kUpChunk;
  const int cnt0 = (int)((mb - first) < kUpChunk ? (mb - first) : kUpChunk);
  const float* src = a.pyr + head + (a.geo.level_off[base_level] + first) * D;
  for (int i = threadIdx.x; i < cnt0 * D; i += blockDim.x) s_a[i] = src[i];
  __syncthreads();
  const int32_t hi = a.L < base_level + kUpLevels ? a.L : base_level + kUpLevels;
  build_levels_in_lds<D>(s_a, s_b, cnt0, first, base_level, hi, a, head);
}

hipError_t launch_build_pyramid(const Problem& p, const void* k, float* pyr, hipStream_t stream) {
  const int64_t plane = (int64_t)p.B * p.Hkv * p.geo.rows * p.D;
  _Float16* f16 = reinterpret_cast<_Float16*>(pyr + plane);
  int32_t* ex = reinterpret_cast<int32_t*>(f16 + plane);
  PyrArgs a{k, pyr, f16, ex, p.N, p.cap, p.B * p.Hkv, p.C, p.L, p.geo};
  const int64_t M1 = level_rows(p.N, p.C, 1);
  const int64_t leaf_blocks = (int64_t)a.BH * ((M1 + kLeafChunk - 1) / kLeafChunk);
  hipError_t err = hipSuccess;
  auto leaf = [&](auto tp, auto dc) {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value;
    PISA_LAUNCH("pyr_leaf", stream, (pyr_leaf_kernel<T, D>), dim3((unsigned)leaf_blocks), dim3(256), 0, a);
    err = hipGetLastError();
    for (int32_t lb = 1 + kLeafLevels; err == hipSuccess && lb < p.L; lb += kUpLevels) {
      const int64_t mb = level_rows(p.N, p.C, lb);
      const int64_t blocks = (int64_t)a.BH * ((mb + kUpChunk - 1) / kUpChunk);
      PISA_LAUNCH("pyr_up", stream, (pyr_up_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, a, lb);
      err = hipGetLastError();
    }
  };
  const bool bf = p.dtype == 1;
  if (p.D == 64) {
    if (bf) leaf(static_cast<uint16_t*>(nullptr), std::integral_constant<int, 64>{});
    else leaf(static_cast<float*>(nullptr), std::integral_constant<int, 64>{});
  } else if (p.D == 128) {
    if (bf) leaf(static_cast<uint16_t*>(nullptr), std::integral_constant<int, 128>{});
    else leaf(static_cast<float*>(nullptr), std::integral_constant<int, 128>{});
  } else {
    return hipErrorInvalidValue;
  }
  return err;
}

}  // namespace pisa
