// Device helpers shared by the PISA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace pisa {

constexpr int kWave = 64;

// For MFMA kernels: at least two waves per SIMD, so at most 256 registers per
// lane.  Within that budget the compiler keeps MFMA accumulators in ordinary
// VGPRs; with the 512-register budget of one wave per SIMD it places them in
// AGPRs and copies every result out with v_accvgpr_read.
#define PISA_MFMA_REGS __attribute__((amdgpu_waves_per_eu(2)))
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// Power-of-two exponent e of a row whose largest magnitude is mx, such that
// mx * 2^-e lies in [2^14, 2^15): the row scaled by 2^-e fits fp16 with full
// relative precision (block floating point; scaling by 2^-e is exact).
__device__ __forceinline__ int row_exponent(float mx) {
  if (!(mx > 0.f)) return 0;
  int e;
  frexpf(mx, &e);  // mx = m * 2^e, m in [0.5, 1)
  return e - 15;
}
__device__ __forceinline__ _Float16 to_f16_scaled(float x, int e) { return (_Float16)ldexpf(x, -e); }

// ---- element access: T is float (fp32) or uint16_t (bf16 bits) ----------
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* out) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Streaming (nontemporal) 16-byte store and load: data written once and read
// once much later (partial records, outputs) marked so that it does not
// displace the cached working set of the kernel that writes or reads it.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void* p, const void* src) {
  __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(p));
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8_nt(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{x.x, x.y, x.z, x.w};
}

// load8 with streaming loads (rows read once)
template <typename T>
__device__ __forceinline__ void load8_nt(const T* p, float* out) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = load16_nt(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const uint4 a = load16_nt(p), b = load16_nt(p + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(w[i]);
  }
}

// 8 consecutive elements of a row, as loaded (16 or 32 bytes), unpacked later
template <typename T>
struct Row8 {
  uint4 v[sizeof(T) == 2 ? 1 : 2];
  __device__ __forceinline__ void load(const T* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    v[0] = q[0];
    if constexpr (sizeof(T) == 4) v[1] = q[1];
  }
  // a streaming load (data read once)
  __device__ __forceinline__ void load_nt(const T* p) {
    v[0] = load16_nt(p);
    if constexpr (sizeof(T) == 4) v[1] = load16_nt(p + 4);
  }
  __device__ __forceinline__ void get(float* out) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t wv[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(wv[i] << 16);
        out[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
      }
    } else {
      const uint32_t wv[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(wv[i]);
    }
  }
};

template <typename T>
__device__ __forceinline__ float load1(const T* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store1(T* p, float v);
template <>
__device__ __forceinline__ void store1<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// ---- wave-level primitives ------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Orders LDS traffic between lanes of one wave (no cross-wave effect).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// x from lane (lane ^ M): a DPP quad permutation for M = 1, 2 (no LDS
// traffic), ds_bpermute otherwise
template <int M>
__device__ __forceinline__ float shfl_xor_dpp(float x) {
  if constexpr (M == 1)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  else if constexpr (M == 2)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  else
    return __shfl_xor(x, M);
}
// sum over aligned groups of W consecutive lanes (W a power of two <= 16)
template <int W>
__device__ __forceinline__ float lane_group_sum(float x) {
  if constexpr (W >= 2) x += shfl_xor_dpp<1>(x);
  if constexpr (W >= 4) x += shfl_xor_dpp<2>(x);
  if constexpr (W >= 8) x += shfl_xor_dpp<4>(x);
  if constexpr (W >= 16) x += shfl_xor_dpp<8>(x);
  return x;
}

// reductions inside aligned groups of `W` lanes (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// 32-bit x from lane (lane ^ m) for a compile-time m after unrolling: DPP for
// m = 1, 2 (quad permutations) and m = 8 (rotation of a 16-lane row by 8,
// which is lane ^ 8 in either rotation direction); ds_bpermute otherwise.
// Lane l's value and lane (l ^ M)'s (M = 16 or 32), in a lane-dependent
// order (for commutative reductions), by the gfx950 permlane swaps: a VALU
// exchange between rows with no LDS round trip.
template <int M>
__device__ __forceinline__ void xor_pair(float x, float& a, float& b) {
  static_assert(M == 16 || M == 32, "rows of 16 or halves of 32 lanes");
  const unsigned u = __float_as_uint(x);
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one per row)
__device__ __forceinline__ float rows_max(float x) {
  float a, b;
  xor_pair<16>(x, a, b);
  xor_pair<32>(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum(float x) {
  float a, b;
  xor_pair<16>(x, a, b);
  xor_pair<32>(a + b, a, b);
  return a + b;
}

// 32-bit x from lane (lane ^ m) for m = 1, 2, 4, 8 (a constant after
// unrolling) by DPP within a row of 16 lanes: quad permutations for 1 and 2;
// for 4, banks 0 and 2 of the row read lane + 4 (row_shl:4) and banks 1 and 3
// lane - 4 (row_shr:4); for 8, a rotation of the row by 8.  No LDS traffic.
__device__ __forceinline__ uint32_t xor_lane_dpp(uint32_t x, int m) {
  const int v = (int)x;
  if (m == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if (m == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if (m == 8) return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror:8
  const int t = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);           // row_shl:4, banks 0, 2
  return (uint32_t)__builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false);        // row_shr:4, banks 1, 3
}

// The 64-bit values of lane l and of lane l ^ m (m a power of two below 64,
// a constant after unrolling) as (a, b): for m < 16, a is the lane's own
// value; for m = 16, 32 the gfx950 permlane swaps exchange whole rows (or
// halves) and the order of the two depends on the lane, which a
// compare-exchange that keeps the larger or the smaller does not see.
__device__ __forceinline__ void xor_pair_u64(uint64_t v, int m, uint64_t& a, uint64_t& b) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  if (m == 16 || m == 32) {
    uint32_t l0, l1, h0, h1;
    if (m == 16) {
      const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
      const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
      l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
    } else {
      const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
    }
    a = ((uint64_t)h0 << 32) | l0;
    b = ((uint64_t)h1 << 32) | l1;
  } else {
    a = v;
    b = ((uint64_t)xor_lane_dpp(hi, m) << 32) | xor_lane_dpp(lo, m);
  }
}

// 2^x for x <= 0 (or -inf) on the hardware exp unit alone, without the
// library's denormal-range fix-up: a result that would be denormal flushes to
// zero, which changes nothing where every use adds it to a term >= 1 (the
// running maximum's own 2^0) or scales a value by it.
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// log(exp(a) + exp(b)) with -inf handled
__device__ __forceinline__ float lse2(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + __logf(__expf(a - m) + __expf(b - m));
}

// ---- total order of every top-K: score descending, then index ascending ---
// 64-bit key, larger = better.  Invalid entries use key 0.
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t score_key(float score, int32_t idx) {
  return ((uint64_t)float_order(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) {
  return (int32_t)(0xFFFFFFFFu - (uint32_t)key);
}
__device__ __forceinline__ float key_score(uint64_t key) { return float_from_order((uint32_t)(key >> 32)); }
// key ordering a kept set by index ascending, carrying the score
__device__ __forceinline__ uint64_t index_key(int32_t idx, float score) {
  return ((uint64_t)(0xFFFFFFFFu - (uint32_t)idx) << 32) | float_order(score);
}
__device__ __forceinline__ int32_t index_key_index(uint64_t key) {
  return (int32_t)(0xFFFFFFFFu - (uint32_t)(key >> 32));
}
__device__ __forceinline__ float index_key_score(uint64_t key) { return float_from_order((uint32_t)key); }

// Bitonic sort inside aligned groups of N lanes (N a power of two <= 64);
// lanes [0, N) end in descending order (other groups alternate direction).
// Each compare-exchange takes the pair (own, partner) from xor_pair_u64 and
// keeps the larger where take_max holds, else the smaller: one 64-bit
// compare, a mask operation and two selects.
template <int N>
__device__ __forceinline__ uint64_t group_sort_desc(uint64_t key) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t x, y;
      xor_pair_u64(key, j, x, y);
      const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
      key = ((x > y) == take_max) ? x : y;
    }
  }
  return key;
}

// Bitonic sort of one 64-bit key per lane, descending across the wave
// (lane 0 ends with the largest key).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key) { return group_sort_desc<kWave>(key); }

// The K largest keys of lanes [0, 2K) land in lanes [0, K), in no particular
// order: sort both K-lane halves (opposite directions) and keep the larger of
// each pair (lane, lane + K) there (lanes [K, 2K) keep the smaller).  K a
// power of two <= 32.
template <int K>
__device__ __forceinline__ uint64_t top_half(uint64_t key) {
  key = group_sort_desc<K>(key);
  uint64_t x, y;
  xor_pair_u64(key, K, x, y);
  return (((lane_id() & K) == 0) == (x > y)) ? x : y;
}

// ---- pyramid geometry (capacity layout, see pisa.h) -----------------------
__host__ __device__ __forceinline__ int64_t level_rows(int64_t n, int32_t C, int32_t l) {
  // M_l(n) = ceil(n / (C * 2^(l-1)))
  const int64_t span = (int64_t)C << (l - 1);
  return (n + span - 1) / span;
}
__host__ __device__ __forceinline__ int32_t num_levels(int64_t n, int32_t C) {
  int64_t m = (n + C - 1) / C;
  int32_t L = 1;
  while (m > 1) {
    m = (m + 1) >> 1;
    ++L;
  }
  return L;
}

constexpr int kMaxLevels = 40;

// Per-call pyramid geometry passed to kernels by value.
struct PyrGeom {
  int64_t level_off[kMaxLevels + 1];  // first row of level l (1-based) in a head
  int64_t rows;                       // rows per (b, h) head (capacity layout)
  int32_t levels_cap;                 // L(cap)
};

// ---- MFMA tiles -----------------------------------------------------------
// One 16x16 output tile accumulated over a 32-wide slice of the contraction.
// Fragment convention (both dtypes): lane l feeds row/column (l % 16) and
// eight contraction elements chosen by the caller for lane group l / 16; A and
// B must use the same choice.  Output: lane l holds rows 4*(l/16)+i, column
// l % 16, i = 0..3.
__device__ __forceinline__ floatx4 mma16x16x32(const float* a8, const float* b8, floatx4 acc) {
  // fp32 inputs: eight K=4 MFMAs, step i pairs element i of every lane group
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a8[i], b8[i], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ floatx4 mma16x16x32(const bf16x8 a, const bf16x8 b, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16x16x32(const halfx8 a, const halfx8 b, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// ---- MFMA operand fragments (8 contraction elements per lane) ---------------
template <typename T>
struct Frag;
template <>
struct Frag<uint16_t> {
  bf16x8 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  // a streaming load (rows read once)
  __device__ __forceinline__ void load_nt(const uint16_t* p) {
    const uint4 u = load16_nt(p);
    v = *reinterpret_cast<const bf16x8*>(&u);
  }
  // elements 0..3 from p0, 4..7 from p1 (each 8-byte aligned)
  __device__ __forceinline__ void load4x2(const uint16_t* p0, const uint16_t* p1) {
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    const uint4 u = {a.x, a.y, b.x, b.y};
    v = *reinterpret_cast<const bf16x8*>(&u);
  }
  // round eight fp32 values to bf16 (nearest even)
  __device__ __forceinline__ void set(const float* x) {
    const uint4 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    v = *reinterpret_cast<const bf16x8*>(&u);
  }
  __device__ __forceinline__ void zero() {
    const uint4 z = {0u, 0u, 0u, 0u};
    v = *reinterpret_cast<const bf16x8*>(&z);
  }
};
template <>
struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) { load8<float>(p, v); }
  __device__ __forceinline__ void load_nt(const float* p) {
    const uint4 a = load16_nt(p), b = load16_nt(p + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  }
  __device__ __forceinline__ void load4x2(const float* p0, const float* p1) {
    const float4 a = *reinterpret_cast<const float4*>(p0);
    const float4 b = *reinterpret_cast<const float4*>(p1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void set(const float* x) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
};
__device__ __forceinline__ floatx4 mma(const Frag<uint16_t>& a, const Frag<uint16_t>& b, floatx4 acc) {
  return mma16x16x32(a.v, b.v, acc);
}
__device__ __forceinline__ floatx4 mma(const Frag<float>& a, const Frag<float>& b, floatx4 acc) {
  return mma16x16x32(a.v, b.v, acc);
}

}  // namespace pisa
