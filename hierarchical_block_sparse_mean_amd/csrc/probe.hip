// Measurement probe (not part of the method): the rate at which the GPU
// serves the gathers that stage-1 routing makes below its LDS stage.  Stage 1
// gathers, per scored level, tiles of 16 child summary rows (fp16, d
// elements) at scattered row indices of one KV head's table: eight lanes load
// each 128-byte piece of a row (eight rows per load), the tile goes to the
// wave's LDS tile (row pitch d + 8) and is read back in the MFMA operand
// layout.  This kernel does the same at pseudo-random rows of a table sized
// like those levels, from persistent workgroups of 16 waves mapped to heads as
// stage 1 maps them, and nothing else: its rate is the ceiling stage 1's
// gathers are measured against.
#include "../../include/pisa.h"
#include "kernels.h"

namespace pisa {

constexpr int kProbeWaves = 16;
constexpr int kProbeUnroll = 4;  // tiles gathered per loop trip (tiles_per_wave is a multiple)

template <int D>
__global__ __launch_bounds__(kProbeWaves* kWave) void probe_gather_kernel(const _Float16* __restrict__ table,
                                                                          int64_t rows_per_head, int32_t heads,
                                                                          int64_t tiles, uint32_t* __restrict__ sink) {
  constexpr int NS = D / 32;      // loads per tile (16 rows x D fp16, 1 KB each)
  constexpr int PITCH = D + 8;    // LDS row pitch (fp16)
  __shared__ __align__(16) _Float16 s_tile[kProbeWaves][16 * PITCH];
  const int w = threadIdx.x / kWave, lane = lane_id(), g = lane >> 4, col = lane & 15;
  const int h = (int)(blockIdx.x % (unsigned)heads);
  const _Float16* hb = table + (int64_t)h * rows_per_head * D;
  _Float16* tile = s_tile[w];
  uint32_t x0 = ((uint32_t)blockIdx.x * kProbeWaves + (uint32_t)w) * 2654435761u + 1u;
  uint32_t acc = 0u;
  for (int64_t i = 0; i < tiles; ++i) {
    // row of tile slot `slot`: a pseudo-random index < rows_per_head
    const uint32_t xt = x0 * 1664525u + (uint32_t)i * 1013904223u;
    halfx8 gv[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int slot = (lane >> 3) + 8 * (st & 1);
      const uint32_t r = (((xt + (uint32_t)slot * 40503u) * 2246822519u) >> 8) % (uint32_t)rows_per_head;
      gv[st] = *reinterpret_cast<const halfx8*>(hb + (int64_t)r * D + 64 * (st >> 1) + 8 * (lane & 7));
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
      *reinterpret_cast<halfx8*>(tile + ((lane >> 3) + 8 * (st & 1)) * PITCH + 64 * (st >> 1) + 8 * (lane & 7)) =
          gv[st];
    wave_sync();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const halfx8 f = *reinterpret_cast<const halfx8*>(tile + col * PITCH + 32 * st + 8 * g);
      const uint4 bits = *reinterpret_cast<const uint4*>(&f);
      acc ^= bits.x ^ bits.y ^ bits.z ^ bits.w;
    }
    wave_sync();
    x0 = x0 * 747796405u + 2891336453u;
  }
  sink[((int64_t)blockIdx.x * kProbeWaves + w) * kWave + lane] = acc;
}

// Streaming probe (not part of the method): the HBM rate of plain 16-byte
// streams, the ceiling the memory-bound kernels are compared with.  mode 0
// reads `bytes` of src with streaming (nontemporal) loads, each thread
// folding its 16-byte pieces into one word of sink; mode 1 copies src to dst;
// unrolled by 8 so every lane keeps eight 16-byte loads in flight, grid-stride
// over the buffer (the highest read rate here came from one workgroup per
// compute unit: about 7.1 TB/s, against about 6 TB/s with sixteen).
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void probe_stream_kernel(const uint4* __restrict__ src,
                                                                      uint4* __restrict__ dst, int64_t n16,
                                                                      int32_t mode, uint32_t* __restrict__ sink) {
  const int64_t tid = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * kStreamThreads;
  uint32_t acc = 0u;
  int64_t i = tid;
  for (; i + (kStreamUnroll - 1) * nthreads < n16; i += kStreamUnroll * nthreads) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = mode == 1 ? src[i + u * nthreads] : load16_nt(src + i + u * nthreads);
    if (mode == 1) {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) dst[i + u * nthreads] = v[u];
    } else {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  for (; i < n16; i += nthreads) {
    const uint4 v = src[i];
    if (mode == 1) dst[i] = v;
    else acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (mode == 0) sink[tid] = acc;
}

}  // namespace pisa

extern "C" pisa_status pisa_probe_stream(const void* src, void* dst, int64_t bytes, int32_t mode,
                                         int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || bytes < 16 || bytes % 16 != 0 || workgroups < 1 || (mode != 0 && mode != 1) ||
      (mode == 1 && dst == nullptr) || (mode == 0 && sink == nullptr) ||
      (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return PISA_ERR_INVALID_ARG;
  PISA_LAUNCH("probe_stream", stream, pisa::probe_stream_kernel, dim3((unsigned)workgroups),
              dim3(pisa::kStreamThreads), 0, static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16,
              mode, sink);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

extern "C" pisa_status pisa_probe_gather(const void* table, int64_t rows_per_head, int32_t heads, int32_t D,
                                         int32_t workgroups, int64_t tiles_per_wave, uint32_t* sink,
                                         hipStream_t stream) {
  if (table == nullptr || sink == nullptr || rows_per_head < 1 || rows_per_head > INT32_MAX || heads < 1 ||
      workgroups < 1 || tiles_per_wave < 1 || tiles_per_wave % pisa::kProbeUnroll != 0 || (D != 64 && D != 128))
    return PISA_ERR_INVALID_ARG;
  const dim3 grid((unsigned)workgroups), block(pisa::kProbeWaves * pisa::kWave);
  const _Float16* t = static_cast<const _Float16*>(table);
  if (D == 128)
    PISA_LAUNCH("probe_gather", stream, pisa::probe_gather_kernel<128>, grid, block, 0, t, rows_per_head, heads,
                tiles_per_wave, sink);
  else
    PISA_LAUNCH("probe_gather", stream, pisa::probe_gather_kernel<64>, grid, block, 0, t, rows_per_head, heads,
                tiles_per_wave, sink);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}
