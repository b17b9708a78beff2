/*
 * synth.c - seeded, counter-based synthetic inputs (host only).
 *
 * This file draws random numbers and rounds them to storage types. It holds
 * none of the attention method's arithmetic: both the CPU oracle and the GPU
 * path consume the exact bytes it produces.
 *
 * Generator, from its published definitions:
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): the n-th output from state s0 is
 *     mix64(s0 + n * 0x9E3779B97F4A7C15) with the 64-bit finaliser below, so
 *     any element can be drawn directly from its index (counter-based).
 *   - Stream key: base(seed, stream) = mix64(mix64(seed) ^ (stream * C2)),
 *     C2 = 0xD1B54A32D192ED03; word(i) = mix64(base + (i + 1) * GAMMA).
 *   - Uniform: u(i) = ((word(i) >> 11) + 0.5) * 2^-53, strictly inside (0, 1).
 *   - Normal: Box and Muller (1958). Element n uses the pair p = n / 2:
 *     r = sqrt(-2 ln u(2p)), theta = 2 pi u(2p + 1); even n -> r cos(theta),
 *     odd n -> r sin(theta). Evaluated in double.
 *   - Rounding: to float32 by C's round-to-nearest-even conversion; to
 *     bfloat16 by round-to-nearest-even applied directly to the double
 *     (one rounding, no double rounding through float32).
 *
 * Every function is deterministic for a given (seed, stream, index) whatever
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL
#define C2 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * C2));
}

static inline double uniform_at(uint64_t base, uint64_t i) {
  uint64_t w = mix64(base + (i + 1) * GAMMA);
  return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t base, uint64_t n) {
  uint64_t p = n >> 1;
  double u1 = uniform_at(base, 2 * p);
  double u2 = uniform_at(base, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (n & 1) ? r * sin(th) : r * cos(th);
}

/* Round a double to bfloat16 (8 significant bits), nearest-even, in one step.
 * Finite inputs whose magnitude lies in float32's normal range or is zero are
 * rounded exactly; larger values saturate to +-inf as a float conversion
 * would. */
static inline uint16_t round_bf16(double x) {
  uint64_t bits;
  memcpy(&bits, &x, 8);
  if ((bits & 0x7FFFFFFFFFFFFFFFULL) == 0) return (uint16_t)((bits >> 48) & 0x8000);
  /* keep 1 + 7 fraction bits of the double's 52: round away the low 45 bits */
  uint64_t lsb = (bits >> 45) & 1ULL;
  bits += 0x00000FFFFFFFFFFFULL + lsb; /* half of the dropped unit, minus 1 */
  bits &= ~0x00001FFFFFFFFFFFULL;
  double y;
  memcpy(&y, &bits, 8);
  float f = (float)y; /* exact: y has at most 8 significant bits */
  uint32_t fb;
  memcpy(&fb, &f, 4);
  return (uint16_t)(fb >> 16);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start,
                       int64_t n, double* out) {
  uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = uniform_at(base, start + (uint64_t)i);
}

/* Fill out[0..n) with normal values start .. start+n-1. Each Box-Muller pair
 * is evaluated once and both of its members are stored when in range. */
#define NORMAL_FILL(STORE)                                                    \
  uint64_t base = stream_base(seed, stream);                                  \
  if (n <= 0) return;                                                         \
  uint64_t p0 = start >> 1, p1 = (start + (uint64_t)n - 1) >> 1;              \
  _Pragma("omp parallel for schedule(static)")                                \
  for (int64_t pp = 0; pp <= (int64_t)(p1 - p0); ++pp) {                      \
    uint64_t p = p0 + (uint64_t)pp;                                           \
    double r = sqrt(-2.0 * log(uniform_at(base, 2 * p)));                     \
    double th = 6.283185307179586476925286766559 * uniform_at(base, 2 * p + 1); \
    uint64_t e = 2 * p;                                                       \
    if (e >= start) { int64_t i = (int64_t)(e - start); STORE(i, r * cos(th)); } \
    if (e + 1 < start + (uint64_t)n) {                                        \
      int64_t i = (int64_t)(e + 1 - start); STORE(i, r * sin(th));            \
    }                                                                         \
  }

#define STORE_F64(i, v) out[i] = (v)
#define STORE_F32(i, v) out[i] = (float)(v)
#define STORE_BF16(i, v) out[i] = round_bf16(v)

void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start,
                      int64_t n, double* out) {
  NORMAL_FILL(STORE_F64)
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start,
                      int64_t n, float* out) {
  NORMAL_FILL(STORE_F32)
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start,
                       int64_t n, uint16_t* out) {
  NORMAL_FILL(STORE_BF16)
}

/* Single element, for spot checks of the counter-based definition. */
double synth_normal_one(uint64_t seed, uint64_t stream, uint64_t index) {
  return normal_at(stream_base(seed, stream), index);
}

void synth_round_bf16(const double* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(x[i]);
}

void synth_round_f32(const double* x, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)x[i];
}
