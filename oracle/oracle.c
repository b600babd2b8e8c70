/*
 * oracle.c — plain CPU reference of the routed-MoE expert layer (TEST INFRASTRUCTURE ONLY:
 * loaded by the tests, the smoke check and the benchmark's CPU-baseline leg, never by the GPU
 * library, with which it shares no code).
 *
 * What the pages fix: a layer holds 512 experts and each token is routed to 10 of them
 * ("Strata vs Llama.cpp vs vLLM", transcript at 08:23; "Local AI Is Now 6x Faster on Your PC",
 * key technological idea); the expert matrix multiply works on low-bit block-quantized weights
 * that are dequantized during the multiply ("Two-Day Port, 8x Faster Prefill: Strata Engine
 * Benchmarked", Where Strata Is Fast; "Strata vs Llama.cpp vs vLLM", transcript at 04:12).
 * The pages print no router formula, FFN form or bit layout.  This file writes out the
 * library's own definitions (softmax top-k routing with ties to the lower index, SwiGLU experts,
 * the Q2/Q3 32-weight block formats, the weighted sum) one step at a time, in fp64, in the
 * order the definition states them, with no blocking, fusion or reordering.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE binary32: widen by shifting the bits up (exact). */
double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int exp = (bits >> 10) & 0x1F;
  int frac = bits & 0x3FF;
  double v;
  if (exp == 0) {
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
  } else if (exp == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp(1.0 + (double)frac / 1024.0, exp - 15);
  }
  return sign ? -v : v;
}

/*
 * Code of weight i (0..31) of one block.
 * 2-bit format: codes packed 16 per little-endian 32-bit word; weight i is in word i/16 at
 * bits 2*(i%16) and 2*(i%16)+1.
 * 3-bit format: the block's 12 bytes form one little-endian 96-bit integer; weight i is at
 * bits 3*i .. 3*i+2.
 */
int32_t oracle_code(int32_t fmt, const uint8_t* blk, int32_t i) {
  if (fmt == 2) {
    const uint8_t* p = blk + 4 * (i / 16);
    uint32_t word = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                    ((uint32_t)p[3] << 24);
    return (int32_t)((word >> (2 * (i % 16))) & 3u);
  }
  int32_t code = 0;
  for (int32_t b = 0; b < 3; ++b) {
    int32_t bit = 3 * i + b;
    code |= ((blk[bit / 8] >> (bit % 8)) & 1) << b;
  }
  return code;
}

/* w = d * (q - c0), c0 = 1.5 for 2-bit codes and 3.5 for 3-bit codes. */
void oracle_dequant_block(int32_t fmt, const uint8_t* blk, uint16_t scale, double out[32]) {
  double d = oracle_f16_to_f64(scale);
  double c0 = (fmt == 2) ? 1.5 : 3.5;
  for (int32_t i = 0; i < 32; ++i) out[i] = d * ((double)oracle_code(fmt, blk, i) - c0);
}

static int64_t code_bytes(int32_t fmt) { return fmt == 2 ? 8 : 12; }

/* rows x K matrix stored as codes [rows][K/32][cb] and scales [rows][K/32]. */
void oracle_dequant_matrix(int32_t fmt, const uint8_t* codes, const uint16_t* scales, int64_t rows,
                           int64_t K, double* out) {
  int64_t nb = K / 32, cb = code_bytes(fmt);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      oracle_dequant_block(fmt, codes + (r * nb + b) * cb, scales[r * nb + b], out + r * K + b * 32);
}

/*
 * Router (the pages: each token goes to 10 of 512 experts, and the routers sit on the GPU:
 * "Strata vs Llama.cpp vs vLLM", transcript 08:23 and 09:28).  Definition: softmax over all
 * logits, keep the k largest probabilities, renormalise them to sum to one.  Softmax is
 * monotone, so the k largest probabilities belong to the k largest logits; selection is made on
 * the fp32 logits by k rounds of arg-max, expert a beating b iff l_a > l_b or (l_a == l_b and
 * a < b).  The renormalised weights are exp(l_j - m) / sum_i exp(l_i - m) over the k picks,
 * m = the largest logit (the full softmax denominator cancels).
 */
void oracle_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, double* w) {
  char* taken = (char*)malloc((size_t)E);
  for (int32_t t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || (double)l[e] > (double)l[best]) best = e; /* equal: keep the lower index */
      }
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    double m = (double)l[ids[(int64_t)t * k]];
    double den = 0.0;
    for (int32_t j = 0; j < k; ++j) den += exp((double)l[ids[(int64_t)t * k + j]] - m);
    for (int32_t j = 0; j < k; ++j)
      w[(int64_t)t * k + j] = exp((double)l[ids[(int64_t)t * k + j]] - m) / den;
  }
  free(taken);
}

/*
 * Grouping of the T*k (token, slot) pairs by expert, slot s = t*k + j: counts per expert, the
 * exclusive prefix sum of the counts, and each expert's slots listed in ascending slot order.
 */
void oracle_permute(const int32_t* ids, int32_t T, int32_t E, int32_t k, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos) {
  int64_t S = (int64_t)T * k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < S; ++s) counts[ids[s]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t s = 0; s < S; ++s) {
    int32_t p = fill[ids[s]]++;
    sorted_slot[p] = (int32_t)s;
    slot_pos[s] = p;
  }
  free(fill);
}

/*
 * One expert on one token: g = W_g x, u = W_u x, a = SiLU(g) * u with SiLU(z) = z / (1 + e^-z),
 * out = W_d a.  x is the token's bf16 activation row widened exactly.  a_row may be NULL.
 */
void oracle_expert_ffn(const oracle_weights* w, int32_t e, const uint16_t* x_row, double* out_row,
                       double* a_row) {
  int64_t H = w->H, I = w->I, cb = code_bytes(w->fmt);
  int64_t nbh = H / 32, nbi = I / 32;
  double* x = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  double blk[32];
  for (int64_t h = 0; h < H; ++h) x[h] = oracle_bf16_to_f64(x_row[h]);
  const uint8_t* gc = w->gate_codes + (int64_t)e * I * nbh * cb;
  const uint8_t* uc = w->up_codes + (int64_t)e * I * nbh * cb;
  const uint16_t* gs = w->gate_scales + (int64_t)e * I * nbh;
  const uint16_t* us = w->up_scales + (int64_t)e * I * nbh;
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int64_t b = 0; b < nbh; ++b) {
      oracle_dequant_block(w->fmt, gc + (n * nbh + b) * cb, gs[n * nbh + b], blk);
      for (int32_t i = 0; i < 32; ++i) g += blk[i] * x[b * 32 + i];
    }
    for (int64_t b = 0; b < nbh; ++b) {
      oracle_dequant_block(w->fmt, uc + (n * nbh + b) * cb, us[n * nbh + b], blk);
      for (int32_t i = 0; i < 32; ++i) u += blk[i] * x[b * 32 + i];
    }
    a[n] = g / (1.0 + exp(-g)) * u;
  }
  const uint8_t* dc = w->down_codes + (int64_t)e * H * nbi * cb;
  const uint16_t* ds = w->down_scales + (int64_t)e * H * nbi;
  for (int64_t h = 0; h < H; ++h) {
    double o = 0.0;
    for (int64_t b = 0; b < nbi; ++b) {
      oracle_dequant_block(w->fmt, dc + (h * nbi + b) * cb, ds[h * nbi + b], blk);
      for (int32_t i = 0; i < 32; ++i) o += blk[i] * a[b * 32 + i];
    }
    out_row[h] = o;
  }
  if (a_row) memcpy(a_row, a, sizeof(double) * (size_t)I);
  free(a);
  free(x);
}

/* y[t] = sum over j = 0..k-1 (ascending) of w[t][j] * expert_out[t*k + j]. */
void oracle_combine(const double* expert_out, const double* w, int32_t T, int32_t k, int32_t H,
                    double* y) {
  for (int32_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j)
        acc += w[(int64_t)t * k + j] * expert_out[((int64_t)t * k + j) * H + h];
      y[(int64_t)t * H + h] = acc;
    }
}

/*
 * The whole layer in the definition's order: route, group slots by expert, run every expert on
 * the tokens of its segment, weighted sum.  Optional outputs (NULL to skip): ids [T][k],
 * w [T][k], expert_out [T*k][H] (slot order), a [T*k][I] (slot order).  Returns 0, or -1 if
 * memory runs out.
 */
int32_t oracle_layer(const oracle_weights* w, const uint16_t* x, const float* logits, int32_t T,
                     int32_t k, double* y, int32_t* ids_out, double* w_out, double* expert_out,
                     double* a_out) {
  int64_t S = (int64_t)T * k, H = w->H, I = w->I;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  double* rw = (double*)malloc(sizeof(double) * (size_t)S);
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)w->E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(w->E + 1));
  int32_t* sorted_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* slot_pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  double* out = expert_out ? expert_out : (double*)malloc(sizeof(double) * (size_t)(S * H));
  if (!ids || !rw || !counts || !offsets || !sorted_slot || !slot_pos || !out) return -1;
  oracle_route(logits, T, w->E, k, ids, rw);
  oracle_permute(ids, T, w->E, k, counts, offsets, sorted_slot, slot_pos);
  for (int32_t e = 0; e < w->E; ++e)
    for (int32_t p = offsets[e]; p < offsets[e + 1]; ++p) {
      int64_t s = sorted_slot[p];
      int64_t t = s / k;
      oracle_expert_ffn(w, e, x + t * H, out + s * H, a_out ? a_out + s * I : NULL);
    }
  oracle_combine(out, rw, T, k, (int32_t)H, y);
  if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)S);
  if (w_out) memcpy(w_out, rw, sizeof(double) * (size_t)S);
  if (!expert_out) free(out);
  free(slot_pos); free(sorted_slot); free(offsets); free(counts); free(rw); free(ids);
  return 0;
}

/*
 * The layer's output for a subset of token rows only (tokens are independent in the layer:
 * each row's routing reads only its own logits and each expert only its own token's x).
 * y_rows [n_rows][H].  Returns 0, or -1 if memory runs out.
 */
int32_t oracle_layer_rows(const oracle_weights* w, const uint16_t* x, const float* logits,
                          int32_t T, int32_t k, const int32_t* rows, int32_t n_rows, double* y_rows) {
  int64_t H = w->H;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* rw = (double*)malloc(sizeof(double) * (size_t)k);
  double* out = (double*)malloc(sizeof(double) * (size_t)(k * H));
  if (!ids || !rw || !out) return -1;
  (void)T;
  for (int32_t r = 0; r < n_rows; ++r) {
    int64_t t = rows[r];
    oracle_route(logits + t * w->E, 1, w->E, k, ids, rw);
    for (int32_t j = 0; j < k; ++j) oracle_expert_ffn(w, ids[j], x + t * H, out + j * H, NULL);
    oracle_combine(out, rw, 1, k, (int32_t)H, y_rows + r * H);
  }
  free(out); free(rw); free(ids);
  return 0;
}

/*
 * Round an fp64 value to bf16, nearest with ties to even, in one step: bf16 keeps 8 significant
 * bits (exponent range as binary32).  v = m * 2^e with m in [0.5, 1); the kept value is
 * rint(m * 2^8) * 2^(e - 8) (rint rounds half to even in the default rounding mode).  Values
 * below the smallest normal binary32 keep fewer bits, as the format's subnormals do.
 */
static uint16_t bf16_from_f64(double v) {
  int e;
  double m = frexp(v, &e);
  int keep = 8;
  if (e - 1 < -126) keep = 8 - (-126 - (e - 1)); /* subnormal range of the format */
  double r = keep >= 0 ? ldexp(rint(ldexp(m, keep)), e - keep) : 0.0;
  float f = (float)r; /* exact: r has at most 8 significant bits and is in binary32 range */
  uint32_t u;
  memcpy(&u, &f, 4);
  if (r == 0.0 && signbit(v)) u = 0x80000000u;
  return (uint16_t)(u >> 16);
}

/*
 * RMSNorm with unit gain for the layer stack: x = bf16(h / sqrt(mean(h^2) + eps)), eps inside
 * the square root.  The mean of squares and the quotient are formed in fp64 and each quotient is
 * rounded once, straight to bf16 (nearest, ties to even).
 */
void oracle_rmsnorm(const float* h, int32_t T, int32_t H, double eps, uint16_t* x) {
  for (int32_t t = 0; t < T; ++t) {
    const float* r = h + (int64_t)t * H;
    double ss = 0.0;
    for (int32_t i = 0; i < H; ++i) ss += (double)r[i] * (double)r[i];
    double den = sqrt(ss / (double)H + eps);
    for (int32_t i = 0; i < H; ++i) x[(int64_t)t * H + i] = bf16_from_f64((double)r[i] / den);
  }
}

/*
 * Router projection: logits[t][e] = sum over h (ascending) of x[t][h] * W_r[e][h], with x (the
 * layer input after RMSNorm) and W_r [E][H] in bf16, widened exactly.  The pages place the
 * routers on the GPU beside the experts ("Strata - the details", How it works / memory tiers;
 * "Strata vs Llama.cpp vs vLLM", transcript at 09:28) and give no formula; a dense linear map
 * from the hidden state to one logit per expert is this library's definition.
 */
void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int32_t T, int32_t H, int32_t E,
                          double* logits) {
  for (int32_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += oracle_bf16_to_f64(x[(int64_t)t * H + h]) * oracle_bf16_to_f64(wr[(int64_t)e * H + h]);
      logits[(int64_t)t * E + e] = acc;
    }
}

/*
 * Shared expert on every token: g = W_sg x, u = W_su x, a = SiLU(g) * u, out = W_sd a, with dense
 * bf16 weights W_sg, W_su [Is][H] and W_sd [H][Is] widened exactly.  The pages list shared experts
 * among what stays on the GPU ("Strata - the details", How it works / memory tiers; "Strata vs
 * Llama.cpp vs vLLM", transcript at 09:28); the SwiGLU form, the same as a routed expert's but
 * dense and unscaled, is this library's definition.  out [T][H].
 */
void oracle_shared_expert(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                          const uint16_t* wd, int32_t T, int32_t H, int32_t Is, double* out) {
  double* a = (double*)malloc(sizeof(double) * (size_t)Is);
  for (int32_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + (int64_t)t * H;
    for (int32_t n = 0; n < Is; ++n) {
      double g = 0.0, u = 0.0;
      for (int32_t h = 0; h < H; ++h) g += oracle_bf16_to_f64(wg[(int64_t)n * H + h]) * oracle_bf16_to_f64(xr[h]);
      for (int32_t h = 0; h < H; ++h) u += oracle_bf16_to_f64(wu[(int64_t)n * H + h]) * oracle_bf16_to_f64(xr[h]);
      a[n] = g / (1.0 + exp(-g)) * u;
    }
    for (int32_t h = 0; h < H; ++h) {
      double o = 0.0;
      for (int32_t n = 0; n < Is; ++n) o += oracle_bf16_to_f64(wd[(int64_t)h * Is + n]) * a[n];
      out[(int64_t)t * H + h] = o;
    }
  }
  free(a);
}

/*
 * Expert usage statistics.  The pages' engine keeps a running distribution of how often each
 * expert is used and treats the most-used ones as hot (video transcript on unbiasedbob.com, 7:47
 * to 7:58; "Strata - the details", How it works / memory tiers).  This library's statistic is the
 * plainest one: usage[e] += the number of (token, slot) pairs routed to expert e, accumulated
 * over calls in 64-bit integers.
 */
void oracle_usage_update(const int32_t* ids, int32_t T, int32_t k, int32_t E, uint64_t* usage) {
  for (int64_t s = 0; s < (int64_t)T * k; ++s) {
    const int32_t e = ids[s];
    if (e >= 0 && e < E) usage[e] += 1;
  }
}

/*
 * Hotness order: order[r] is the expert of rank r, experts sorted by usage, most used first,
 * equal usage broken by the lower expert index.  Written as E rounds of picking the largest
 * not-yet-picked count (selection), the definition read literally.
 */
void oracle_usage_rank(const uint64_t* usage, int32_t E, int32_t* order) {
  char* taken = (char*)calloc((size_t)E, 1);
  for (int32_t r = 0; r < E; ++r) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || usage[e] > usage[best]) best = e;
    }
    order[r] = best;
    taken[best] = 1;
  }
  free(taken);
}
