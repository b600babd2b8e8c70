/*
 * Seeded synthetic inputs for the MoE expert layer: one counter-based generator shared by the
 * CPU oracle's tests and the GPU benchmark, so both see byte-identical inputs.  This file holds
 * no arithmetic of the layer itself: it only draws random bytes, normal deviates and the
 * storage roundings that define the inputs (fp32 -> bf16 and -> fp16, round to nearest even).
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3", SC 2011): a 128-bit counter and a 64-bit key go through ten rounds of two 32x32->64
 * multiplies with xor mixing, the key bumped by the Weyl constants between rounds.
 *
 * Stream layout: key = {stream, seed_lo32}, counter = {i_lo, i_hi, seed_hi32, 0}.  Counter i
 * yields 16 bytes (4 little-endian words) for byte streams, and four normal deviates for normal
 * streams (two Box-Muller pairs from words (0,1) and (2,3)).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void mi_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block_at(uint64_t seed, uint32_t stream, uint64_t i, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), (uint32_t)(seed >> 32), 0u};
  uint32_t key[2] = {stream, (uint32_t)seed};
  mi_philox4x32_10(ctr, key, out);
}

/* Uniform in the open interval (0, 1) from the top 24 bits of a word. */
static inline double unit_open(uint32_t w) { return ((double)(w >> 8) + 0.5) * (1.0 / 16777216.0); }

static inline void box_muller(uint32_t a, uint32_t b, double* z0, double* z1) {
  const double two_pi = 6.283185307179586476925286766559;
  double r = sqrt(-2.0 * log(unit_open(a)));
  double th = two_pi * unit_open(b);
  *z0 = r * cos(th);
  *z1 = r * sin(th);
}

static inline double normal_at(uint64_t seed, uint32_t stream, uint64_t n) {
  uint32_t w[4];
  block_at(seed, stream, n >> 2, w);
  double z[4];
  box_muller(w[0], w[1], &z[0], &z[1]);
  box_muller(w[2], w[3], &z[2], &z[3]);
  return z[n & 3];
}

/* fp32 -> bf16, round to nearest even (inputs here are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + rounding) >> 16);
}

/* fp32 -> IEEE binary16, round to nearest even, with subnormals; overflow saturates to inf. */
static inline uint16_t f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t mag = u & 0x7FFFFFFFu;
  if (mag >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (mag > 0x7F800000u ? 0x200u : 0u));
  int32_t exp = (int32_t)(mag >> 23) - 127;
  uint32_t mant = mag & 0x7FFFFFu;
  if (exp > 15) return (uint16_t)(sign | 0x7C00u);
  if (exp >= -14) {
    /* normal half: keep 10 mantissa bits of 23, round the dropped 13 */
    uint32_t h = ((uint32_t)(exp + 15) << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* may carry into exponent */
    return (uint16_t)(sign | h);
  }
  if (exp < -25) return (uint16_t)sign; /* below half the smallest subnormal */
  /* subnormal half: value = m * 2^-24 with m = full significand >> shift */
  uint32_t full = mant | 0x800000u;
  int shift = -exp - 1; /* 14..24 : full * 2^(exp-23) / 2^-24 = full >> (-exp-1) */
  uint32_t h = full >> shift;
  uint32_t rem = full & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (h & 1u))) h += 1u;
  return (uint16_t)(sign | h);
}

void mi_fill_bytes(uint64_t seed, uint32_t stream, uint8_t* out, uint64_t n) {
  uint64_t nblk = (n + 15) / 16;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)nblk; ++i) {
    uint32_t w[4];
    block_at(seed, stream, (uint64_t)i, w);
    uint8_t b[16];
    for (int j = 0; j < 4; ++j) {
      b[4 * j + 0] = (uint8_t)(w[j]);
      b[4 * j + 1] = (uint8_t)(w[j] >> 8);
      b[4 * j + 2] = (uint8_t)(w[j] >> 16);
      b[4 * j + 3] = (uint8_t)(w[j] >> 24);
    }
    uint64_t base = (uint64_t)i * 16;
    uint64_t cnt = (n - base < 16) ? (n - base) : 16;
    memcpy(out + base, b, (size_t)cnt);
  }
}

/* out[i] = fp32(scale * N_i + bias[i % bias_len]) (bias may be NULL). */
void mi_fill_normal_f32(uint64_t seed, uint32_t stream, double scale, const double* bias,
                        int64_t bias_len, float* out, uint64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    double z = scale * normal_at(seed, stream, (uint64_t)i);
    if (bias) z += bias[i % bias_len];
    out[i] = (float)z;
  }
}

/* out[i] = bf16_RNE(fp32(N_i)) */
void mi_fill_normal_bf16(uint64_t seed, uint32_t stream, uint16_t* out, uint64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = f32_to_bf16((float)normal_at(seed, stream, (uint64_t)i));
}

/* out[i] = fp16_RNE(fp32(mult * |N_i|)) */
void mi_fill_abs_normal_f16(uint64_t seed, uint32_t stream, double mult, uint16_t* out, uint64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = f32_to_f16((float)(mult * fabs(normal_at(seed, stream, (uint64_t)i))));
}

/* Seeded permutation of 0..n-1 (Fisher-Yates, index j = floor(u * (i+1)) with u a 32-bit word). */
void mi_permutation(uint64_t seed, uint32_t stream, int32_t* perm, int32_t n) {
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint32_t w[4];
    block_at(seed, stream, (uint64_t)i, w);
    int32_t j = (int32_t)(((uint64_t)w[0] * (uint64_t)(i + 1)) >> 32);
    int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
}

/* Exposed for tests of the storage roundings. */
void mi_f32_to_bf16_array(const float* in, uint16_t* out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}
void mi_f32_to_f16_array(const float* in, uint16_t* out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_f16(in[i]);
}
