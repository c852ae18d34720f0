/*
 * Seeded synthetic inputs shared by the HIP path's tests/benchmarks and by the CPU oracle.
 *
 * This file holds no arithmetic of the method itself: it only turns (seed, stream, row) counters into
 * bfloat16 values distributed approximately N(0,1), standing in for KV rows written by prefill and for
 * decode queries (the pages use real model KV; none is available, so seeded synthetic rows of the same
 * width replace it).
 *
 * Generator: every row is a pure function of (seed, domain, a, b, row) so results do not depend on the
 * thread count or on which rows are generated first.
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
 *     mixes the counters into one 64-bit word per pair of output values;
 *   - the upper and lower 24-bit fields of that word give two uniforms in (0,1);
 *   - the Box-Muller transform (Box and Muller 1958) maps them to two standard normals;
 *   - each float32 normal is rounded to bfloat16 with round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t row_key(uint64_t seed, uint32_t domain, int64_t a, int64_t b, int64_t row) {
  uint64_t h = mix64(seed + GOLDEN * ((uint64_t)domain + 1u));
  h = mix64(h ^ (GOLDEN * ((uint64_t)a + 0x1000u)));
  h = mix64(h ^ (GOLDEN * ((uint64_t)b + 0x2000u)));
  h = mix64(h ^ (GOLDEN * ((uint64_t)row + 0x3000u)));
  return h;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void fill_one_row(uint16_t* dst, uint64_t key, int32_t row_elems) {
  const float two_pi = 6.28318530717958647692f;
  for (int32_t e = 0; e < row_elems; e += 2) {
    uint64_t w = mix64(key + GOLDEN * (uint64_t)(e / 2 + 1));
    float u1 = ((float)(w >> 40) + 0.5f) * (1.0f / 16777216.0f);
    float u2 = (float)((w >> 16) & 0xFFFFFFu) * (1.0f / 16777216.0f);
    float r = sqrtf(-2.0f * logf(u1));
    float t = two_pi * u2;
    dst[e] = f32_to_bf16_rne(r * cosf(t));
    if (e + 1 < row_elems) dst[e + 1] = f32_to_bf16_rne(r * sinf(t));
  }
}

/* Rows [first_row, first_row + count) of stream (seed, domain, a, b), row_elems bf16 each, into dst. */
void synth_rows_bf16(uint16_t* dst, uint64_t seed, uint32_t domain, int64_t a, int64_t b,
                     int64_t first_row, int64_t count, int32_t row_elems, int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static, 256) num_threads(nthreads)
  for (int64_t i = 0; i < count; ++i)
    fill_one_row(dst + i * (int64_t)row_elems, row_key(seed, domain, a, b, first_row + i), row_elems);
}

/* Rows at arbitrary positions pos[count] of stream (seed, domain, a, b) into dst[count][row_elems]. */
void synth_rows_at_bf16(uint16_t* dst, uint64_t seed, uint32_t domain, int64_t a, int64_t b,
                        const int32_t* pos, int64_t count, int32_t row_elems, int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static, 64) num_threads(nthreads)
  for (int64_t i = 0; i < count; ++i)
    fill_one_row(dst + i * (int64_t)row_elems, row_key(seed, domain, a, b, pos[i]), row_elems);
}
