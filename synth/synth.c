/* Seeded synthetic inputs: a counter-based SplitMix64 stream, Box-Muller
 * normals, fp32 -> bf16 round-to-nearest-even, and integer-uniform lengths.
 *
 * This file holds no attention arithmetic. It serves both the fp64 oracle and
 * the HIP path, which receive the same bits.
 *
 * SplitMix64 is the generator of G. L. Steele, D. Lea and C. H. Flood, "Fast
 * splittable pseudorandom number generators" (OOPSLA 2014): state advances by
 * the odd constant 0x9e3779b97f4a7c15 and each output is the state passed
 * through the Stafford "mix13" finaliser. Because state n is seed + n*gamma,
 * output n can be computed directly from n, so every element of a tensor is a
 * pure function of (seed, stream, index) and any slice can be regenerated
 * without the rest. Normals use the Box-Muller transform (Box and Muller,
 * 1958), cosine branch, one normal per two uniforms.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stddef.h>

#define GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

/* n-th output (n >= 0) of the SplitMix64 sequence started from `seed`:
 * the generator first advances the state, then mixes it. */
uint64_t synth_splitmix64_at(uint64_t seed, uint64_t n) {
  return mix64(seed + (n + 1) * GAMMA);
}

/* Per-tensor key: one SplitMix64 output of the user seed, offset by stream. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed + (stream + 1) * GAMMA) ^ (stream * 0xd1b54a32d192ed03ULL);
}

static inline double uniform_open0(uint64_t x) { /* (0, 1] */
  return ((double)(x >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}
static inline double uniform_closed0(uint64_t x) { /* [0, 1) */
  return (double)(x >> 11) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t a = mix64(key + (2 * i + 1) * GAMMA);
  uint64_t b = mix64(key + (2 * i + 2) * GAMMA);
  double u1 = uniform_open0(a), u2 = uniform_closed0(b);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* fp32 -> bf16 bits, round to nearest, ties to even. NaN stays NaN. */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[j] = element (offset + j) of the stream: float(stddev * N) rounded to
 * bf16. Element indices are global, so slices of one tensor agree with the
 * whole tensor generated at once. */
void synth_normal_bf16(uint16_t* out, uint64_t offset, uint64_t count,
                       uint64_t seed, uint64_t stream, double stddev) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)count; ++j) {
    float f = (float)(stddev * normal_at(key, offset + (uint64_t)j));
    out[j] = f32_to_bf16(f);
  }
}

void synth_normal_f32(float* out, uint64_t offset, uint64_t count,
                      uint64_t seed, uint64_t stream, double stddev) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = (float)(stddev * normal_at(key, offset + (uint64_t)j));
}

/* Integers uniform on the inclusive range [lo, hi] (multiply-shift, 32 bits). */
void synth_uniform_i32(int32_t* out, uint64_t count, int32_t lo, int32_t hi,
                       uint64_t seed, uint64_t stream) {
  uint64_t key = stream_key(seed, stream);
  uint64_t range = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
  for (uint64_t j = 0; j < count; ++j) {
    uint64_t x = mix64(key + (j + 1) * GAMMA) >> 32;
    out[j] = (int32_t)((int64_t)lo + (int64_t)((x * range) >> 32));
  }
}

/* bf16 bits of an fp32 array, RNE; used to round host-made values. */
void synth_round_bf16(const float* in, uint16_t* out, uint64_t count) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)count; ++j) out[j] = f32_to_bf16(in[j]);
}
