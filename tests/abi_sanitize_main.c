/*
 * The C ABI's host-side argument checks and size queries under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Test infrastructure only: tests/test_oracle_sanitize.py compiles
 * the library's sources host-only (no GPU code) with the host sanitizers, links this driver and
 * runs it on the CPU.  Every compute call below fails validation or is a T = 0 no-op, so no HIP
 * call is made; the fake device addresses are never dereferenced.  The size queries are swept
 * over shapes up to the 32-bit limits, where a signed overflow would be reported.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "strata_moe.h"

#define A ((void*)(uintptr_t)0x10000)   /* 16-byte aligned stand-in address */
#define MIS ((void*)(uintptr_t)0x10004) /* misaligned stand-in */

static int g_bad = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    g_bad = 1;
  }
}

static strata_moe_weights weights(int fmt, int E, int H, int I, const void* ptr) {
  strata_moe_weights w;
  memset(&w, 0, sizeof w);
  w.fmt = fmt;
  w.num_experts = E;
  w.hidden = H;
  w.inter = I;
  w.gate_codes = ptr;
  w.up_codes = ptr;
  w.gate_scales = (const uint16_t*)ptr;
  w.up_scales = (const uint16_t*)ptr;
  w.down_codes = ptr;
  w.down_scales = (const uint16_t*)ptr;
  w.stats = (const strata_moe_expert_stats*)ptr;
  return w;
}

int main(void) {
  const int OK = STRATA_OK, INVAL = STRATA_ERR_INVALID_ARGUMENT, UNSUP = STRATA_ERR_UNSUPPORTED,
            WS = STRATA_ERR_WORKSPACE_TOO_SMALL;
  for (int st = 0; st < 8; ++st)
    if (!strata_status_string((strata_status)st)) g_bad = 1;
  if (strcmp(strata_status_string((strata_status)99), "unknown status") != 0) g_bad = 1;

  /* size queries over the whole accepted range and past it */
  const int32_t Ts[] = {-1, 0, 1, 4, 8, 9, 32, 33, 8192, 65536, 1 << 20, INT_MAX};
  const int32_t Es[] = {-1, 0, 1, 64, 512, 1024, 1025, INT_MAX};
  const int32_t ks[] = {-1, 0, 1, 10, 16, 17, INT_MAX};
  const int32_t Hs[] = {0, 256, 3072, 65536, INT_MAX};
  const int32_t Is[] = {0, 128, 768, 65536, INT_MAX};
  volatile size_t sink = 0;
  for (size_t a = 0; a < sizeof Ts / sizeof Ts[0]; ++a)
    for (size_t b = 0; b < sizeof Es / sizeof Es[0]; ++b)
      for (size_t c = 0; c < sizeof ks / sizeof ks[0]; ++c) {
        sink += strata_moe_permute_workspace_bytes(Ts[a], Es[b], ks[c]);
        for (size_t d = 0; d < sizeof Hs / sizeof Hs[0]; ++d)
          for (size_t e = 0; e < sizeof Is / sizeof Is[0]; ++e) {
            sink += strata_moe_workspace_bytes(Ts[a], Es[b], ks[c], Hs[d], Is[e]);
            sink += strata_moe_residual_workspace_bytes(Ts[a], Es[b], ks[c], Hs[d], Is[e]);
            sink += strata_moe_block_workspace_bytes(Ts[a], Es[b], ks[c], Hs[d], Is[e], Is[e]);
          }
      }
  for (size_t a = 0; a < sizeof Ts / sizeof Ts[0]; ++a)
    for (size_t e = 0; e < sizeof Is / sizeof Is[0]; ++e)
      sink += strata_moe_shared_workspace_bytes(Ts[a], Is[e]);
  sink += strata_moe_decode_static_max_bytes();
  (void)sink;

  /* routing and the permutation */
  expect(strata_moe_route(A, 4, 8, 9, A, A, NULL), INVAL, "route k > E");
  expect(strata_moe_route(A, -1, 512, 10, A, A, NULL), INVAL, "route T < 0");
  expect(strata_moe_route(A, 4, 2048, 10, A, A, NULL), UNSUP, "route E > 1024");
  expect(strata_moe_route(MIS, 4, 512, 10, A, A, NULL), INVAL, "route misaligned");
  expect(strata_moe_route(NULL, 0, 512, 10, NULL, NULL, NULL), OK, "route T = 0");
  const size_t pw = strata_moe_permute_workspace_bytes(8192, 512, 10);
  expect(strata_moe_permute(A, 8192, 512, 10, A, A, A, A, A, pw - 1, NULL), WS, "permute ws");
  expect(strata_moe_permute(A, 8192, 512, 10, A, A, NULL, A, A, pw, NULL), INVAL, "permute null");
  expect(strata_moe_permute(A, INT_MAX, 1024, 16, A, A, A, A, A, pw, NULL) == OK, 0,
         "permute T = INT_MAX accepted");

  /* weights, the layer entry points and the static-scratch decode */
  const size_t ws = strata_moe_workspace_bytes(8192, 512, 10, 3072, 768);
  strata_moe_weights w = weights(2, 512, 3072, 768, A);
  expect(strata_moe_layer(&w, A, A, 8192, 10, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws - 1, NULL),
         WS, "layer ws");
  expect(strata_moe_layer(&w, A, A, 8192, 0, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws, NULL),
         INVAL, "layer k = 0");
  expect(strata_moe_layer(NULL, A, A, 16, 4, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws, NULL),
         INVAL, "layer null weights");
  strata_moe_weights bad_fmt = weights(4, 512, 3072, 768, A);
  expect(strata_moe_layer(&bad_fmt, A, A, 16, 4, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws, NULL),
         INVAL, "layer fmt");
  strata_moe_weights bad_h = weights(2, 512, 3000, 768, A);
  expect(strata_moe_layer(&bad_h, A, A, 16, 4, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws, NULL),
         INVAL, "layer H");
  strata_moe_weights bad_ptr = weights(2, 512, 3072, 768, MIS);
  expect(strata_moe_layer(&bad_ptr, A, A, 16, 4, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws, NULL),
         INVAL, "layer misaligned weights");
  strata_moe_weights big = weights(2, INT_MAX, INT_MAX, INT_MAX, A);
  expect(strata_moe_layer(&big, A, A, INT_MAX, 16, A, 0, NULL, NULL, NULL, NULL, NULL, A, ws, NULL)
             == OK, 0, "layer at the 32-bit limits accepted");
  expect(strata_moe_expert_ffn(&w, A, 8192, 10, A, A, A, A, ws - 1, NULL), WS, "expert_ffn ws");
  expect(strata_moe_decode(&w, A, A, 9, 10, A, 0, NULL, NULL, A, ws, NULL), UNSUP, "decode T = 9");
  expect(strata_moe_decode_static(&w, A, A, 9, 10, A, 0, NULL, NULL, NULL), UNSUP,
         "decode_static T = 9");
  expect(strata_moe_decode_static(&bad_fmt, A, A, 4, 10, A, 0, NULL, NULL, NULL), INVAL,
         "decode_static fmt");
  expect(strata_moe_decode_static(&w, NULL, A, 4, 10, A, 0, NULL, NULL, NULL), INVAL,
         "decode_static null x");
  expect(strata_moe_decode_static(&w, NULL, NULL, 0, 10, NULL, 0, NULL, NULL, NULL), OK,
         "decode_static T = 0");
  const size_t rws = strata_moe_residual_workspace_bytes(4, 512, 10, 3072, 768);
  expect(strata_moe_layer_residual(&w, A, A, 4, 10, NAN, A, rws, NULL), INVAL, "residual eps NaN");
  expect(strata_moe_layer_residual(&w, A, A, 4, 10, 1e-6f, A, rws - 1, NULL), WS, "residual ws");
  const size_t bws = strata_moe_block_workspace_bytes(4, 512, 10, 3072, 768, 768);
  expect(strata_moe_block(&w, A, 4, 10, A, A, A, A, 96, A, A, 0, A, bws, NULL), UNSUP, "block Is");
  expect(strata_moe_block(&w, NULL, 0, 10, A, A, A, A, 768, NULL, A, 0, A, bws, NULL), OK,
         "block T = 0");
  expect(strata_moe_weight_stats(&w, MIS, NULL), INVAL, "weight_stats misaligned");

  /* combine, RMSNorm, repack, dense layers, usage statistics */
  expect(strata_moe_combine(A, A, 4, 10, 3072, NULL, 0, NULL), INVAL, "combine null y");
  expect(strata_moe_combine(A, A, 0, 10, 3072, A, 0, NULL), OK, "combine T = 0");
  expect(strata_moe_rmsnorm(A, 4, 3072, -1.0f, A, NULL), INVAL, "rmsnorm eps");
  expect(strata_moe_rmsnorm(A, 4, 3071, 1e-6f, A, NULL), UNSUP, "rmsnorm H");
  char* B = (char*)A + (1 << 30);
  const uint16_t* As = (const uint16_t*)((char*)A + 4096);
  uint16_t* Bs = (uint16_t*)(B + 4096);
  expect(strata_moe_pack_matrix(2, 1, 64, 64, A, As, (char*)A + 512, Bs, NULL), INVAL,
         "pack overlap");
  expect(strata_moe_pack_matrix(2, INT_MAX, INT_MAX, INT_MAX, A, As, B, Bs, NULL) == OK, 0,
         "pack at the 32-bit limits accepted");
  expect(strata_moe_router_logits(A, A, 4, 3000, 512, A, NULL), UNSUP, "router H");
  const size_t sws = strata_moe_shared_workspace_bytes(8192, 768);
  expect(strata_moe_shared_expert(A, A, A, A, 8192, 3072, 768, A, 0, A, sws - 1, NULL), WS,
         "shared ws");
  expect(strata_moe_usage_update(A, 4, 10, 2048, A, NULL), UNSUP, "usage E");
  expect(strata_moe_usage_rank(A, 512, MIS, NULL), INVAL, "usage_rank misaligned");

  if (g_bad) {
    fprintf(stderr, "C ABI sanitizer run: FAILED\n");
    return 1;
  }
  printf("C ABI sanitizer run: ok\n");
  return 0;
}
