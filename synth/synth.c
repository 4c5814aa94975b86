/*
 * synth.c -- seeded synthetic inputs shared by the tests, the oracle checks and
 * the benchmark.  This file holds no arithmetic of the approximate multiply: it
 * only turns (seed, stream, element index) into numbers.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), keyed by splitmix64 (Steele, Lea,
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA'14).
 * Counter-based, so every element is a pure function of its index and the
 * output does not depend on the thread count.
 *
 *   uniform   u = ((x >> 11) + 1) * 2^-53  in (0, 1]   (x = 64 bits of Philox)
 *   normals   Box-Muller in double: r = sqrt(-2 ln u1), z0 = r cos(2 pi u2),
 *             z1 = r sin(2 pi u2)
 *   weights   W = fp16_rne(scale * z)                    (binary16 bits)
 *   acts      v = fp32(scale * z0 / sqrt((z1^2+z2^2+z3^2)/3))  (Student-t, nu=3)
 *
 * Element e of a normal stream uses Philox block e/2, half e%2.  The Philox
 * counter is (block lo, block hi, stream lo, stream hi); the key is the two
 * halves of splitmix64(seed).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static uint64_t splitmix64_next(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    philox_round(c, k);
    if (r != 9) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
  }
  memcpy(out, c, sizeof c);
}

uint64_t synth_splitmix64(uint64_t x) {
  uint64_t s = x;
  return splitmix64_next(&s);
}

static inline void make_key(uint64_t seed, uint32_t key[2]) {
  uint64_t s = seed;
  uint64_t k = splitmix64_next(&s);
  key[0] = (uint32_t)k;
  key[1] = (uint32_t)(k >> 32);
}

/* Two normals from Philox block `blk` of stream `stream`. */
static inline void normal_pair(uint64_t blk, uint64_t stream, const uint32_t key[2],
                               double* z0, double* z1) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)stream,
                     (uint32_t)(stream >> 32)};
  uint32_t o[4];
  synth_philox4x32_10(ctr, key, o);
  uint64_t x1 = ((uint64_t)o[1] << 32) | o[0];
  uint64_t x2 = ((uint64_t)o[3] << 32) | o[2];
  double u1 = (double)((x1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)((x2 >> 11) + 1) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(th);
  *z1 = r * sin(th);
}

/* IEEE-754 binary64 -> binary16, round to nearest even. */
uint16_t synth_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double ax = fabs(x);
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
  if (ax >= 65520.0) return (uint16_t)(sign | 0x7C00u); /* rounds past 65504 */
  if (ax < 0x1.0p-14) {
    /* subnormal range: value = q * 2^-24, scaling by 2^24 is exact */
    double q = nearbyint(ax * 0x1.0p24); /* default rounding mode: to nearest even */
    return (uint16_t)(sign | (uint16_t)q); /* q == 1024 lands on the smallest normal */
  }
  int e;
  double fr = frexp(ax, &e); /* ax = fr * 2^e, fr in [0.5, 1) */
  e -= 1;                    /* ax = (2 fr) * 2^e, 2 fr in [1, 2) */
  double q = nearbyint(fr * 2048.0); /* 1024 .. 2048 */
  if (q >= 2048.0) { q = 1024.0; e += 1; }
  int be = e + 15;
  if (be >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)(be << 10) | (uint16_t)((int)q - 1024));
}

/* count normals z_e, e = first .. first+count-1, of (seed, stream). */
void synth_normals(double* out, int64_t first, int64_t count, uint64_t seed, uint64_t stream) {
  uint32_t key[2];
  make_key(seed, key);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    int64_t e = first + t;
    double z0, z1;
    normal_pair((uint64_t)e >> 1, stream, key, &z0, &z1);
    out[t] = (e & 1) ? z1 : z0;
  }
}

/* fp16 weights: bits of fp16_rne(scale * z_e) for e = 0 .. count-1. */
void synth_weights_f16(uint16_t* out, int64_t count, double scale, uint64_t seed,
                       uint64_t stream) {
  uint32_t key[2];
  make_key(seed, key);
  int64_t blocks = (count + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < blocks; ++b) {
    double z0, z1;
    normal_pair((uint64_t)b, stream, key, &z0, &z1);
    out[2 * b] = synth_f64_to_f16(scale * z0);
    if (2 * b + 1 < count) out[2 * b + 1] = synth_f64_to_f16(scale * z1);
  }
}

/* fp32 Student-t(3) activations: v_i from normals 4i .. 4i+3. */
void synth_student_t3_f32(float* out, int64_t count, double scale, uint64_t seed,
                          uint64_t stream) {
  uint32_t key[2];
  make_key(seed, key);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    double z0, z1, z2, z3;
    normal_pair((uint64_t)(2 * i), stream, key, &z0, &z1);
    normal_pair((uint64_t)(2 * i + 1), stream, key, &z2, &z3);
    double chi = sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
    out[i] = (float)(scale * z0 / chi);
  }
}

/* uniform doubles in (0, 1]: element e uses the first 64 bits of Philox block e. */
void synth_uniforms(double* out, int64_t count, uint64_t seed, uint64_t stream) {
  uint32_t key[2];
  make_key(seed, key);
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < count; ++e) {
    uint32_t ctr[4] = {(uint32_t)e, (uint32_t)((uint64_t)e >> 32), (uint32_t)stream,
                       (uint32_t)(stream >> 32)};
    uint32_t o[4];
    synth_philox4x32_10(ctr, key, o);
    uint64_t x = ((uint64_t)o[1] << 32) | o[0];
    out[e] = (double)((x >> 11) + 1) * 0x1.0p-53;
  }
}
