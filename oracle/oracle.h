/*
 * oracle.h — plain, slow, single-threaded CPU reference of the routed-MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library; the GPU library never links, calls or includes it, and it shares
 * no code, header, table or constant with the GPU library.
 *
 * Arithmetic is IEEE fp64 throughout (inputs widened exactly), summations run sequentially in
 * index order, built with -O2 -ffp-contract=off and no fast-math.  Every function states the
 * definition it writes out; see oracle.c for the citations of the pages.
 */
#ifndef STRATA_ORACLE_H
#define STRATA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_weights {
  int32_t fmt; /* 2 = 2-bit codes (offset 1.5, 8 code bytes per block), 3 = 3-bit (3.5, 12 B) */
  int32_t E, H, I;
  const uint8_t* gate_codes; const uint16_t* gate_scales; /* [E][I][H/32] */
  const uint8_t* up_codes;   const uint16_t* up_scales;   /* [E][I][H/32] */
  const uint8_t* down_codes; const uint16_t* down_scales; /* [E][H][I/32] */
} oracle_weights;

double oracle_bf16_to_f64(uint16_t bits);
double oracle_f16_to_f64(uint16_t bits);
int32_t oracle_code(int32_t fmt, const uint8_t* block_codes, int32_t i);
void oracle_dequant_block(int32_t fmt, const uint8_t* block_codes, uint16_t scale, double out[32]);
void oracle_dequant_matrix(int32_t fmt, const uint8_t* codes, const uint16_t* scales, int64_t rows,
                           int64_t K, double* out);

void oracle_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, double* w);
void oracle_permute(const int32_t* ids, int32_t T, int32_t E, int32_t k, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos);
void oracle_expert_ffn(const oracle_weights* w, int32_t e, const uint16_t* x_row, double* out_row,
                       double* a_row);
void oracle_combine(const double* expert_out, const double* w, int32_t T, int32_t k, int32_t H,
                    double* y);
int32_t oracle_layer(const oracle_weights* w, const uint16_t* x, const float* logits, int32_t T,
                     int32_t k, double* y, int32_t* ids_out, double* w_out, double* expert_out,
                     double* a_out);
int32_t oracle_layer_rows(const oracle_weights* w, const uint16_t* x, const float* logits,
                          int32_t T, int32_t k, const int32_t* rows, int32_t n_rows, double* y_rows);
void oracle_rmsnorm(const float* h, int32_t T, int32_t H, double eps, uint16_t* x);
void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int32_t T, int32_t H, int32_t E,
                          double* logits);
void oracle_shared_expert(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                          const uint16_t* wd, int32_t T, int32_t H, int32_t Is, double* out);
void oracle_usage_update(const int32_t* ids, int32_t T, int32_t k, int32_t E, uint64_t* usage);
void oracle_usage_rank(const uint64_t* usage, int32_t E, int32_t* order);

#ifdef __cplusplus
}
#endif
#endif
