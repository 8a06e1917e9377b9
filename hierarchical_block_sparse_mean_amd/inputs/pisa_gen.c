/*
 * Counter-based synthetic input generator (host C, OpenMP).
 *
 * Holds no arithmetic of the attention method: it only turns (seed, stream,
 * element index) into numbers, so that any slice of any tensor can be
 * regenerated on its own and both the CPU oracle and the GPU library are fed
 * bit-identical inputs.
 *
 *   SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014), used in counter form: draw c of a stream with
 *   key s is mix(s + (c + 1) * GAMMA).
 *   stream key = mix(mix(seed + GAMMA) ^ ((stream + 1) * GAMMA)).
 *   Normal draws: Box-Muller (1958) in double precision, element i uses draws
 *   2i and 2i+1: u1 = ((w1 >> 11) + 1) * 2^-53 in (0, 1],
 *   u2 = (w2 >> 11) * 2^-53 in [0, 1), z = sqrt(-2 ln u1) * cos(2 pi u2).
 *   bf16 outputs: double -> float (round to nearest even) -> bf16 (round to
 *   nearest even on the upper 16 bits).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

uint64_t pisa_gen_stream_key(uint64_t seed, uint64_t stream) {
  return mix(mix(seed + GAMMA) ^ ((stream + 1) * GAMMA));
}

static inline uint64_t draw(uint64_t key, uint64_t c) { return mix(key + (c + 1) * GAMMA); }

static inline double normal_at(uint64_t key, int64_t i) {
  uint64_t w1 = draw(key, 2 * (uint64_t)i);
  uint64_t w2 = draw(key, 2 * (uint64_t)i + 1);
  double u1 = (double)((w1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(w2 >> 11) * 0x1.0p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

void pisa_gen_normal_f64(uint64_t seed, uint64_t stream, int64_t start, int64_t n, double* out) {
  const uint64_t key = pisa_gen_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, start + i);
}

void pisa_gen_normal_f32(uint64_t seed, uint64_t stream, int64_t start, int64_t n, float* out) {
  const uint64_t key = pisa_gen_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)normal_at(key, start + i);
}

void pisa_gen_normal_bf16(uint64_t seed, uint64_t stream, int64_t start, int64_t n,
                          uint16_t* out) {
  const uint64_t key = pisa_gen_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16((float)normal_at(key, start + i));
}

/* Raw 64-bit draws c = start .. start+n-1 of a stream (for index choices). */
void pisa_gen_u64(uint64_t seed, uint64_t stream, int64_t start, int64_t n, uint64_t* out) {
  const uint64_t key = pisa_gen_stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, (uint64_t)(start + i));
}

/* Round doubles to bf16 bits / float (same rounding as the normal draws). */
void pisa_gen_f64_to_bf16(const double* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16((float)in[i]);
}
