/*
 * Seeded synthetic inputs for the decode step: weights, K/V prefixes, token ids.
 *
 * This file is input plumbing shared by the oracle side and the GPU side of the
 * tests and the benchmark. It holds none of the decode step's arithmetic: it only
 * draws numbers.
 *
 * Generator: a counter-based stream. Element pair p of stream (seed, stream) is
 * mix64(key + (p + 1) * GOLDEN), where mix64 is the SplitMix64 output function
 * (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number Generators",
 * OOPSLA 2014) and key = mix64(mix64(seed) ^ (stream * GOLDEN2)). Because every
 * value is a pure function of (seed, stream, index), any slice can be drawn
 * independently and in parallel, and the result does not depend on the thread count.
 *
 * Normals: Box and Muller (1958). The 64-bit draw of pair p is split into two
 * 32-bit uniforms u1, u2 in (0, 1); element 2p = r cos(2 pi u2), element 2p+1 =
 * r sin(2 pi u2), with r = sqrt(-2 ln u1). The value is scaled in double, rounded
 * to float, and for bf16 output rounded from float to bf16 to nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define GOLDEN2 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * GOLDEN2));
}

static inline uint64_t draw(uint64_t key, uint64_t counter) { return mix64(key + (counter + 1) * GOLDEN); }

static inline void normal_pair(uint64_t r, double* z0, double* z1) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = ((double)(r >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(r & 0xFFFFFFFFULL) + 0.5) * (1.0 / 4294967296.0);
  double rad = sqrt(-2.0 * log(u1));
  *z0 = rad * cos(two_pi * u2);
  *z1 = rad * sin(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u); /* NaN stays NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[i] = float(mean + std * N_i) for i in [0, n), N_i the i-th standard normal of the stream. */
void synth_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, double mean, double std) {
  const uint64_t key = stream_key(seed, stream);
  const int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    double z0, z1;
    normal_pair(draw(key, (uint64_t)p), &z0, &z1);
    out[2 * p] = (float)(mean + std * z0);
    if (2 * p + 1 < n) out[2 * p + 1] = (float)(mean + std * z1);
  }
}

/* Same draws as synth_normal_f32, then rounded to bf16 (bit patterns in out). */
void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, double mean, double std) {
  const uint64_t key = stream_key(seed, stream);
  const int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    double z0, z1;
    normal_pair(draw(key, (uint64_t)p), &z0, &z1);
    out[2 * p] = f32_to_bf16_rne((float)(mean + std * z0));
    if (2 * p + 1 < n) out[2 * p + 1] = f32_to_bf16_rne((float)(mean + std * z1));
  }
}

/* out[i] uniform in [lo, hi] (inclusive), i-th draw of the stream. */
void synth_uniform_i64(int64_t* out, int64_t n, uint64_t seed, uint64_t stream, int64_t lo, int64_t hi) {
  const uint64_t key = stream_key(seed, stream);
  const uint64_t span = (uint64_t)(hi - lo) + 1ULL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = lo + (int64_t)(draw(key, (uint64_t)i) % span);
}
