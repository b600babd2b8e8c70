/*
 * Calls every entry point of the CPU oracle (oracle/oracle.c) on small inputs, so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer checks the oracle's own memory accesses
 * and arithmetic.  Test infrastructure only: tests/test_oracle_sanitize.py builds it with gcc
 * and -fsanitize=address,undefined and runs it; any sanitizer report aborts the run.
 *
 * Inputs come from a local LCG: they only need to be in range for the calls, and the values are
 * not compared here (the oracle's pins in tests/test_oracle.py do that).  Both code formats
 * (2-bit, 3-bit) and shapes with a token count that is not a multiple of anything are used, plus
 * the degenerate cases the oracle accepts (k = 1, one expert, T = 0 rows of layer_rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x243F6A8885A308D3ull;

static uint32_t next_u32(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 32);
}

/* uniform in (-1, 1) */
static double next_sym(void) { return ((double)next_u32() + 0.5) / 2147483648.0 - 1.0; }

/* bf16 bits of f (round to nearest even; f is finite here) */
static uint16_t bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* a positive normal fp16 scale in [2^-8, 2^-5) */
static uint16_t small_f16_scale(void) {
  return (uint16_t)(((7u + next_u32() % 3u) << 10) | (next_u32() & 0x3FFu));
}

static void* must_alloc(size_t n) {
  void* p = calloc(n ? n : 1, 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static void fill_bytes(uint8_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)next_u32();
}

static void fill_scales(uint16_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) p[i] = small_f16_scale();
}

static void fill_bf16(uint16_t* p, size_t n, double amp) {
  for (size_t i = 0; i < n; ++i) p[i] = bf16_bits((float)(amp * next_sym()));
}

static int check_finite(const double* v, size_t n, const char* what) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(v[i])) {
      fprintf(stderr, "%s[%zu] is not finite\n", what, i);
      return 1;
    }
  return 0;
}

/* One layer shape through every layer-level entry point. */
static int run_layer_case(int32_t fmt, int32_t E, int32_t H, int32_t I, int32_t T, int32_t k) {
  const size_t cb = fmt == 2 ? 8 : 12; /* code bytes per 32-weight block */
  const size_t gblocks = (size_t)E * I * (H / 32), dblocks = (size_t)E * H * (I / 32);
  uint8_t* gc = must_alloc(gblocks * cb);
  uint8_t* uc = must_alloc(gblocks * cb);
  uint8_t* dc = must_alloc(dblocks * cb);
  uint16_t* gs = must_alloc(gblocks * 2);
  uint16_t* us = must_alloc(gblocks * 2);
  uint16_t* ds = must_alloc(dblocks * 2);
  fill_bytes(gc, gblocks * cb);
  fill_bytes(uc, gblocks * cb);
  fill_bytes(dc, dblocks * cb);
  fill_scales(gs, gblocks);
  fill_scales(us, gblocks);
  fill_scales(ds, dblocks);
  const oracle_weights w = {fmt, E, H, I, gc, gs, uc, us, dc, ds};

  const size_t S = (size_t)T * k;
  uint16_t* x = must_alloc((size_t)T * H * 2);
  float* logits = must_alloc((size_t)T * E * sizeof(float));
  fill_bf16(x, (size_t)T * H, 2.0);
  for (size_t i = 0; i < (size_t)T * E; ++i) logits[i] = (float)(3.0 * next_sym());
  if (T > 1) logits[E] = logits[0]; /* a tie across tokens, and one within token 1 below */
  if (T > 1 && E > 1) logits[E + 1] = logits[E];

  int32_t* ids = must_alloc(S * 4);
  double* rw = must_alloc(S * 8);
  oracle_route(logits, T, E, k, ids, rw);
  int32_t* counts = must_alloc((size_t)E * 4);
  int32_t* offsets = must_alloc((size_t)(E + 1) * 4);
  int32_t* sorted_slot = must_alloc(S * 4);
  int32_t* slot_pos = must_alloc(S * 4);
  oracle_permute(ids, T, E, k, counts, offsets, sorted_slot, slot_pos);

  double* eo = must_alloc(S * H * 8);
  double* a = must_alloc(S * I * 8);
  for (size_t s = 0; s < S; ++s)
    oracle_expert_ffn(&w, ids[s], x + (s / k) * H, eo + s * H, a + s * I);
  double* y = must_alloc((size_t)T * H * 8);
  oracle_combine(eo, rw, T, k, H, y);

  double* y2 = must_alloc((size_t)T * H * 8);
  int32_t* ids2 = must_alloc(S * 4);
  double* rw2 = must_alloc(S * 8);
  double* eo2 = must_alloc(S * H * 8);
  double* a2 = must_alloc(S * I * 8);
  int bad = 0;
  bad |= oracle_layer(&w, x, logits, T, k, y2, ids2, rw2, eo2, a2) != 0;
  bad |= oracle_layer(&w, x, logits, T, k, y2, NULL, NULL, NULL, NULL) != 0;

  int32_t rows[3] = {T - 1, 0, T / 2};
  double* yr = must_alloc(3 * (size_t)H * 8);
  bad |= oracle_layer_rows(&w, x, logits, T, k, rows, 3, yr) != 0;
  bad |= oracle_layer_rows(&w, x, logits, T, k, rows, 0, yr) != 0;

  uint64_t* usage = must_alloc((size_t)E * 8);
  int32_t* order = must_alloc((size_t)E * 4);
  oracle_usage_update(ids, T, k, E, usage);
  oracle_usage_update(ids, T, k, E, usage);
  oracle_usage_rank(usage, E, order);

  bad |= check_finite(y, (size_t)T * H, "combine y");
  bad |= check_finite(y2, (size_t)T * H, "layer y");
  bad |= check_finite(yr, 3 * (size_t)H, "layer_rows y");
  if (memcmp(y, y2, (size_t)T * H * 8) != 0) {
    fprintf(stderr, "layer and step-by-step results differ (fmt %d)\n", fmt);
    bad = 1;
  }

  free(order); free(usage); free(yr); free(a2); free(eo2); free(rw2); free(ids2); free(y2);
  free(y); free(a); free(eo); free(slot_pos); free(sorted_slot); free(offsets); free(counts);
  free(rw); free(ids); free(logits); free(x); free(ds); free(us); free(gs); free(dc); free(uc);
  free(gc);
  return bad;
}

/* Dequantization, conversions, RMSNorm and the dense layers. */
static int run_elementwise_cases(void) {
  int bad = 0;
  for (int32_t fmt = 2; fmt <= 3; ++fmt) {
    const size_t cb = fmt == 2 ? 8 : 12;
    const int64_t rows = 3, K = 96;
    uint8_t* codes = must_alloc((size_t)rows * (K / 32) * cb);
    uint16_t* scales = must_alloc((size_t)rows * (K / 32) * 2);
    fill_bytes(codes, (size_t)rows * (K / 32) * cb);
    fill_scales(scales, (size_t)rows * (K / 32));
    double* out = must_alloc((size_t)rows * K * 8);
    oracle_dequant_matrix(fmt, codes, scales, rows, K, out);
    double blk[32];
    oracle_dequant_block(fmt, codes + cb, scales[1], blk);
    for (int32_t i = 0; i < 32; ++i) {
      const int32_t q = oracle_code(fmt, codes, i);
      if (q < 0 || q > (fmt == 2 ? 3 : 7)) bad = 1;
      if (blk[i] != out[32 + i]) bad = 1;
    }
    free(out); free(scales); free(codes);
  }
  for (uint32_t b = 0; b < 65536; b += 257) {
    (void)oracle_bf16_to_f64((uint16_t)b);
    (void)oracle_f16_to_f64((uint16_t)b);
  }

  const int32_t T = 3, H = 64, E = 5, Is = 32;
  float* h = must_alloc((size_t)T * H * 4);
  for (int32_t i = 0; i < T * H; ++i) h[i] = (float)next_sym();
  for (int32_t i = 0; i < H; ++i) h[(T - 1) * H + i] = 0.0f; /* an all-zero row */
  uint16_t* xr = must_alloc((size_t)T * H * 2);
  oracle_rmsnorm(h, T, H, 1e-6, xr);

  uint16_t* wr = must_alloc((size_t)E * H * 2);
  uint16_t* wg = must_alloc((size_t)Is * H * 2);
  uint16_t* wu = must_alloc((size_t)Is * H * 2);
  uint16_t* wd = must_alloc((size_t)H * Is * 2);
  fill_bf16(wr, (size_t)E * H, 0.1);
  fill_bf16(wg, (size_t)Is * H, 0.1);
  fill_bf16(wu, (size_t)Is * H, 0.1);
  fill_bf16(wd, (size_t)H * Is, 0.1);
  double* lg = must_alloc((size_t)T * E * 8);
  double* so = must_alloc((size_t)T * H * 8);
  oracle_router_logits(xr, wr, T, H, E, lg);
  oracle_shared_expert(xr, wg, wu, wd, T, H, Is, so);
  bad |= check_finite(lg, (size_t)T * E, "router logits");
  bad |= check_finite(so, (size_t)T * H, "shared expert");
  free(so); free(lg); free(wd); free(wu); free(wg); free(wr); free(xr); free(h);
  return bad;
}

int main(void) {
  int bad = run_elementwise_cases();
  bad |= run_layer_case(2, 8, 64, 64, 7, 3);
  bad |= run_layer_case(3, 8, 64, 96, 5, 4);
  bad |= run_layer_case(2, 1, 32, 32, 3, 1); /* one expert, top-1 */
  bad |= run_layer_case(3, 16, 96, 32, 9, 16); /* k = E */
  if (bad) {
    fprintf(stderr, "oracle sanitizer run: FAILED\n");
    return 1;
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
