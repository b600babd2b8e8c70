/*
 * Calls every entry point of the seeded input generator (moe_inputs/gen.c) with lengths that end
 * inside a 16-byte Philox block or a four-deviate group, and with the storage roundings' edge
 * values (subnormal, overflowing and exactly halfway fp32 inputs), so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer checks the generator's memory accesses and
 * integer arithmetic.  Test infrastructure only: tests/test_oracle_sanitize.py builds and runs it.
 * Values are checked by tests/test_inputs.py; here only ranges are.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void mi_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
void mi_fill_bytes(uint64_t seed, uint32_t stream, uint8_t* out, uint64_t n);
void mi_fill_normal_f32(uint64_t seed, uint32_t stream, double scale, const double* bias,
                        int64_t bias_len, float* out, uint64_t n);
void mi_fill_normal_bf16(uint64_t seed, uint32_t stream, uint16_t* out, uint64_t n);
void mi_fill_abs_normal_f16(uint64_t seed, uint32_t stream, double mult, uint16_t* out, uint64_t n);
void mi_permutation(uint64_t seed, uint32_t stream, int32_t* perm, int32_t n);
void mi_f32_to_bf16_array(const float* in, uint16_t* out, uint64_t n);
void mi_f32_to_f16_array(const float* in, uint16_t* out, uint64_t n);

int main(void) {
  int bad = 0;
  const uint32_t ctr[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  const uint32_t key[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
  uint32_t blk[4];
  mi_philox4x32_10(ctr, key, blk);

  const uint64_t lens[] = {0, 1, 3, 15, 16, 17, 37, 1000};
  for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li) {
    const uint64_t n = lens[li];
    const uint64_t seed = 0xFFFFFFFFFFFFFFFFull - li;
    uint8_t* b = malloc(n ? n : 1);
    float* f = malloc((n ? n : 1) * sizeof(float));
    uint16_t* h = malloc((n ? n : 1) * 2);
    uint16_t* g = malloc((n ? n : 1) * 2);
    if (!b || !f || !h || !g) return 2;
    mi_fill_bytes(seed, 7u, b, n);
    const double bias[3] = {0.5, -1.0, 2.0};
    mi_fill_normal_f32(seed, 0xFFFFFFFFu, 1.0, bias, 3, f, n);
    mi_fill_normal_f32(seed, 1u, 2.0, NULL, 0, f, n);
    for (uint64_t i = 0; i < n; ++i)
      if (!isfinite(f[i])) bad = 1;
    mi_fill_normal_bf16(seed, 2u, h, n);
    mi_fill_abs_normal_f16(seed, 3u, 0.02, g, n);
    for (uint64_t i = 0; i < n; ++i)
      if (g[i] & 0x8000u) bad = 1; /* |N| is never negative */
    free(g); free(h); free(f); free(b);
  }

  const int32_t pn[] = {0, 1, 2, 13, 512};
  for (size_t pi = 0; pi < sizeof pn / sizeof pn[0]; ++pi) {
    const int32_t n = pn[pi];
    int32_t* perm = malloc((size_t)(n ? n : 1) * 4);
    char* seen = calloc((size_t)(n ? n : 1), 1);
    if (!perm || !seen) return 2;
    mi_permutation(99u, 5u, perm, n);
    for (int32_t i = 0; i < n; ++i) {
      if (perm[i] < 0 || perm[i] >= n || seen[perm[i]]) bad = 1;
      else seen[perm[i]] = 1;
    }
    free(seen); free(perm);
  }

  const float edge[] = {0.0f, -0.0f, 1e-45f, -1e-45f, 5.96e-8f, 2.98e-8f, 6.1e-5f, 65504.0f,
                        65520.0f, 1e30f, -1e30f, 3.4e38f, 1.0f + 1.0f / 256.0f, 1.00390625f,
                        1.0009765625f, 1.00048828125f, -2.5f};
  const uint64_t ne = sizeof edge / sizeof edge[0];
  uint16_t ob[sizeof edge / sizeof edge[0]], oh[sizeof edge / sizeof edge[0]];
  mi_f32_to_bf16_array(edge, ob, ne);
  mi_f32_to_f16_array(edge, oh, ne);
  if (oh[8] != 0x7C00u || ob[0] != 0u || oh[1] != 0x8000u) bad = 1;

  if (bad) {
    fprintf(stderr, "input generator sanitizer run: FAILED\n");
    return 1;
  }
  printf("input generator sanitizer run: ok\n");
  return 0;
}
