/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file only draws random numbers and rounds them; it holds none of the
 * scoring or eviction arithmetic. Both the CPU oracle and the GPU path take
 * their inputs from here, so the two see bit-identical tensors.
 *
 * Streams: element n of stream `key` is the n-th output of the splitmix64
 * generator started at state `key` (state advances by the golden-ratio
 * increment, output is the splitmix64 finaliser). Because every element is a
 * pure function of (key, n), the result does not depend on how the work is
 * split across threads.
 *
 * Normals: Box-Muller on consecutive output pairs (2p, 2p+1), in double:
 *   u1 = (x >> 11 + 1) * 2^-53 in (0, 1],  u2 = (y >> 11) * 2^-53 in [0, 1)
 *   z0 = sqrt(-2 ln u1) cos(2 pi u2),       z1 = sqrt(-2 ln u1) sin(2 pi u2)
 * Element e takes z0 when e is even and z1 when e is odd.
 *
 * bfloat16: round-to-nearest-even of the fp32 bit pattern (upper 16 bits).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_at(uint64_t key, uint64_t n) {
  return mix64(key + (n + 1) * GOLDEN);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) ^ mix64(stream * 0xD1B54A32D192ED03ULL + 1));
}

void synth_u64(uint64_t key, uint64_t first, int64_t count, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < count; ++e) out[e] = stream_at(key, first + (uint64_t)e);
}

static inline double normal_at(uint64_t key, uint64_t e) {
  const uint64_t p = e >> 1;
  const uint64_t x = stream_at(key, 2 * p);
  const uint64_t y = stream_at(key, 2 * p + 1);
  const double u1 = (double)((x >> 11) + 1) * 0x1.0p-53;
  const double u2 = (double)(y >> 11) * 0x1.0p-53;
  const double r = sqrt(-2.0 * log(u1));
  const double t = 6.283185307179586476925286766559 * u2;
  return (e & 1) ? r * sin(t) : r * cos(t);
}

/* out[e] = (float)(mean + std * z_e), e in [0, count), z from stream `key`
 * starting at element `first`. */
void synth_normal_f32(uint64_t key, uint64_t first, int64_t count, double mean,
                      double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < count; ++e)
    out[e] = (float)(mean + std * normal_at(key, first + (uint64_t)e));
}

void synth_normal_f64(uint64_t key, uint64_t first, int64_t count, double mean,
                      double std, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < count; ++e)
    out[e] = mean + std * normal_at(key, first + (uint64_t)e);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

void synth_f32_to_bf16(const float* in, int64_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < count; ++e) out[e] = f32_to_bf16_rne(in[e]);
}

/* Normal draws rounded straight to bf16: out[e] = bf16(float(mean + std*z)). */
void synth_normal_bf16(uint64_t key, uint64_t first, int64_t count, double mean,
                       double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < count; ++e)
    out[e] = f32_to_bf16_rne(
        (float)(mean + std * normal_at(key, first + (uint64_t)e)));
}
