// Decode / verify path for T <= 8 tokens: bandwidth-bound GEMVs over the touched experts.
//
// The pages verify up to 3 drafted tokens plus one in a single pass over the layers ("Strata - the
// details", How it works / speculation) and note that decode is bound by memory bandwidth
// ("Two-Day Port, 8x Faster Prefill: Strata Engine Benchmarked", Why Prefill Matters).  Every
// touched expert's packed weights are streamed from HBM exactly once and applied to every token
// that picked it, so HBM bytes are the packed size of the distinct touched experts.
//
// Two kernels (a kernel boundary costs ~1.7 us on MI355X; a grid-wide barrier inside one kernel
// costs far more, because the per-XCD L2s must be written back and invalidated):
//  K1 up:   one 16-wave workgroup per CU.  Every workgroup routes all T tokens itself (one wave
//           per token), lists the distinct experts and the (token, slot) pairs of each, and works
//           through a contiguous range of items (distinct expert, 4 rows of I), one wave per
//           item: a = SiLU(g) * u per token, rounded to bf16.  Workgroup 0 publishes the routing
//           for K2 and the caller.
//  K2 down: workgroup b owns rows [b R, (b+1) R) of H (R = H / 256) for ALL distinct experts, so it
//           holds every slot's down output for its rows and forms y = sum_j w_j out_j itself, in
//           slot order: deterministic, and no third launch.
//
// Arithmetic.  Weights enter exactly.  A 2-bit code q is placed into the mantissa of a bf16 whose
// exponent makes it 2 + q * 2^(e-6), e in {0, 2, 4} the bit offset the mask leaves it at, so a
// 16-code word becomes 8 bf16 pairs with 2 shifts and 8 and-or operations.  The activation of that
// pair is staged multiplied by s = 2^(6-e) (exact in bf16), so each v_dot2 product is
// 2 s x + q x; the block's constant part C = sum (2 s + 1.5) x is staged with it, and
//   sum_i (q_i - 1.5) x_i = dot - C,   the block's value = d * (dot - C), d its fp16 scale.
// 3-bit codes: bf16 4 + q/2 with x staged times 2: dot = sum (8 + q) x, C = 11.5 sum x.
// x stays bf16 (the input precision); a is rounded to bf16 between the GEMVs; y is fp32.
//
// Pairing: pair m (m = 0..7) of a 16-value word holds values m and m + 8.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace strata {

constexpr int kUpThreads = 1024;   // K1: 16 waves, one workgroup per CU
constexpr int kDnThreads = 1024;   // K2: 16 waves, one workgroup per CU
constexpr int kGrid = 256;         // one workgroup per CU
constexpr int kDecMaxT = 8;
constexpr int kDecMaxS = 128;      // T * k <= 8 * 16
constexpr int kDecMaxR = 16;       // rows of H per K2 workgroup (H <= 4096)
constexpr int kUpRows = 4;         // rows of I per K1 item: one wave, 16 lanes per row
constexpr int kDnPieces = 9;       // K2: 16-byte pieces of staged a per thread (<= 144 KB of LDS)


// Routes token t (this wave) into LDS.
template <int NPL>
STRATA_DEVICE void route_token_npl(const float* __restrict__ logits, int t, int E, int k,
                                   int* ids_s, float* w_s, uint64_t* sel) {
  TokenKeys<NPL> tk;
  load_token_logits<NPL>(logits + (size_t)t * E, E, tk);
  select_token_wave<NPL>(tk, E, k, ids_s + t * k, w_s + t * k, sel);
}

// sel: this wave's 80 uint64 of selection LDS.
STRATA_DEVICE void route_token(const float* __restrict__ logits, int t, int E, int k, int* ids_s,
                               float* w_s, uint64_t* sel) {
  if (E <= 64) route_token_npl<1>(logits, t, E, k, ids_s, w_s, sel);
  else if (E <= 128) route_token_npl<2>(logits, t, E, k, ids_s, w_s, sel);
  else if (E <= 256) route_token_npl<4>(logits, t, E, k, ids_s, w_s, sel);
  else if (E <= 512) route_token_npl<8>(logits, t, E, k, ids_s, w_s, sel);
  else route_token_npl<16>(logits, t, E, k, ids_s, w_s, sel);
}

// ---------------------------------------------------------------------------------------------
// Routing table: distinct experts in order of first appearance among the T*k slots, and for each
// the (token, slot) pairs that picked it.

struct RouteTable {
  int ids[kDecMaxS];
  float w[kDecMaxS];
  int dexp[kDecMaxS];                  // distinct experts
  int dtp[kDecMaxS];                   // tokens per distinct expert
  uint8_t dtok[kDecMaxS][kDecMaxT];    // their tokens
  uint8_t dslot[kDecMaxS][kDecMaxT];   // and slots
  int nd;
};

// The part of the table K2 needs, as K1 publishes it in the workspace.
struct GlobalTable {
  int nd;
  int pad[3];
  int dexp[kDecMaxS];
  int dtp[kDecMaxS];
  uint8_t dslot[kDecMaxS][kDecMaxT];
};

// Clears what build_table accumulates into; must be visible (a barrier) before build_table.
// scratch: E ints of LDS that stay untouched until build_table returns.
template <int NTHREADS>
STRATA_DEVICE void table_clear(RouteTable& rt, int S, int E, int* scratch) {
  for (int e = threadIdx.x; e < E; e += NTHREADS) scratch[e] = 0x7FFFFFFF;
  if (threadIdx.x < S) rt.dtp[threadIdx.x] = 0;
}

// Builds the table from rt.ids (visible to the workgroup) after table_clear.
STRATA_DEVICE void build_table(RouteTable& rt, int T, int k, int* scratch) {
  int* first_slot = scratch;  // per expert: lowest slot that picked it
  __shared__ uint64_t first_mask[kDecMaxS / 64];
  const int S = T * k, q = threadIdx.x;
  const int id = q < S ? rt.ids[q] : 0;
  if (q < S) atomicMin(&first_slot[id], q);
  __syncthreads();
  const int f = q < S ? first_slot[id] : 0;  // the slot that represents this slot's expert
  const uint64_t ball = __ballot(q < S && f == q);
  if ((q & 63) == 0 && (q >> 6) < kDecMaxS / 64) first_mask[q >> 6] = ball;
  __syncthreads();
  if (q < S) {
    // the expert's position in the distinct list: first occurrences before f
    const uint64_t m0 = first_mask[0];
    const int pos = f < 64 ? __popcll(m0 & ((1ull << f) - 1ull))
                           : __popcll(m0) + __popcll(first_mask[1] & ((1ull << (f - 64)) - 1ull));
    if (f == q) rt.dexp[pos] = id;
    // a token picks an expert at most once, and the per-token arithmetic does not depend on the
    // position in the expert's list
    const int idx = atomicAdd(&rt.dtp[pos], 1);
    rt.dtok[pos][idx] = (uint8_t)(q / k);
    rt.dslot[pos][idx] = (uint8_t)q;
  }
  if (q == 0) rt.nd = __popcll(first_mask[0]) + (S > 64 ? __popcll(first_mask[1]) : 0);
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// Staged activations in LDS.  A row of K values is K/64 chunks; chunk ch starts at dword 36 ch
// (32 dwords of pairs and 4 of padding, so that the chunks read together by neighbouring lanes
// start in different LDS banks), word q of the chunk at +8 q, pair m at +m.  The constant part C
// of each 32-value block is a float in a separate array, K/32 per row.

constexpr int kChunkDwords = 36;

// Stages one block (32 values; v holds them in natural order as 16 bf16 pairs) of a row.
template <int FMT>
STRATA_DEVICE void stage_block(const u32x4_t (&v)[4], uint32_t* prow, float* crow, int blk) {
  float c = 0.0f;
#pragma unroll
  for (int ww = 0; ww < 2; ++ww) {
    uint32_t pr[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int ia = 16 * ww + m, ib = ia + 8;  // values m and m + 8 of the word
      const uint32_t da = v[(ia >> 1) >> 2][(ia >> 1) & 3], db = v[(ib >> 1) >> 2][(ib >> 1) & 3];
      const float xa = __uint_as_float((ia & 1) ? (da & 0xFFFF0000u) : (da << 16));
      const float xb = __uint_as_float((ib & 1) ? (db & 0xFFFF0000u) : (db << 16));
      const float s = FMT == 2 ? (m % 3 == 0 ? 64.0f : m % 3 == 1 ? 16.0f : 4.0f) : 2.0f;
      const float coef = FMT == 2 ? 2.0f * s + 1.5f : 11.5f;
      pr[m] = (__float_as_uint(xa * s) >> 16) | (__float_as_uint(xb * s) & 0xFFFF0000u);
      c = __builtin_fmaf(coef, xa, c);
      c = __builtin_fmaf(coef, xb, c);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(prow + kChunkDwords * (blk >> 1) + 8 * (2 * (blk & 1) + ww));
    dst[0] = u32x4_t{pr[0], pr[1], pr[2], pr[3]};
    dst[1] = u32x4_t{pr[4], pr[5], pr[6], pr[7]};
  }
  crow[blk] = c;
}

__host__ __device__ inline size_t staged_row_bytes(int K) { return (size_t)(K / 64) * kChunkDwords * 4 + (size_t)(K / 32) * 4; }

// ---------------------------------------------------------------------------------------------
// Weight rows in the tiled layout: a row's chunk ch (reduction indices 64 ch .. 64 ch + 63, two
// blocks) sits in stage ch of its 4-row group, the stages of one group being consecutive
// (4 rows x 2 cb code bytes and 4 x 2 fp16 scales each).  A lane holds chunks c0, c0 + cstep, ...
// (< nchunk) of one row, at most MC.

template <int FMT>
STRATA_DEVICE const uint8_t* tiled_row_codes(const uint8_t* codes, size_t row, int nchunk) {
  constexpr int CB = FMT == 2 ? 8 : 12;
  return codes + (row >> 2) * nchunk * (8 * CB) + (row & 3) * (2 * CB);
}

STRATA_DEVICE const uint16_t* tiled_row_scales(const uint16_t* scales, size_t row, int nchunk) {
  return scales + (row >> 2) * nchunk * 8 + (row & 3) * 2;
}

template <int FMT, int MC>
struct RowChunks {
  static constexpr int kWords = FMT == 2 ? 4 : 6;  // 32-bit words of code bytes per chunk
  uint32_t w[MC][kWords];
  uint32_t sc[MC];                                 // the chunk's two fp16 block scales
};

// row_codes / row_scales: the row's chunk 0 (tiled_row_codes / tiled_row_scales).
template <int FMT, int MC>
STRATA_DEVICE void load_row_chunks(RowChunks<FMT, MC>& rc, const uint8_t* row_codes,
                                   const uint16_t* row_scales, int nchunk, int c0, int cstep) {
  constexpr int CB = FMT == 2 ? 8 : 12;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int ch = c0 + cstep * i;
    if (ch < nchunk) {
      const uint8_t* cp = row_codes + (size_t)ch * (8 * CB);
      if constexpr (FMT == 2) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp));
        rc.w[i][0] = v[0]; rc.w[i][1] = v[1]; rc.w[i][2] = v[2]; rc.w[i][3] = v[3];
      } else {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t* p = reinterpret_cast<const u32x2_t*>(cp);
        const u32x2_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1),
                      d = __builtin_nontemporal_load(p + 2);
        rc.w[i][0] = a[0]; rc.w[i][1] = a[1]; rc.w[i][2] = b[0]; rc.w[i][3] = b[1];
        rc.w[i][4] = d[0]; rc.w[i][5] = d[1];
      }
      rc.sc[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row_scales + (size_t)ch * 8));
    }
  }
}

// The chunks of two rows (codes0 / scales0 and codes1 / scales1: each row's chunk 0, from
// tiled_row_codes / tiled_row_scales), loaded chunk by chunk, both rows' words of a chunk
// together: row_dots works chunk by chunk, so the counter wait before chunk i then covers chunks
// 0..i only.  Used by K2, whose lane groups start computing as their only unit's data lands
// (K2 12.04 -> 11.64 us); K1's waves, which take items one after another, keep the row order.
template <int FMT, int MC>
STRATA_DEVICE void load_row_pair_chunks(RowChunks<FMT, MC> (&rc)[2], const uint8_t* codes0,
                                        const uint16_t* scales0, const uint8_t* codes1,
                                        const uint16_t* scales1, int nchunk, int c0, int cstep) {
  constexpr int CB = FMT == 2 ? 8 : 12;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int ch = c0 + cstep * i;
    if (ch < nchunk) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t* cp = (j ? codes1 : codes0) + (size_t)ch * (8 * CB);
        if constexpr (FMT == 2) {
          const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp));
          rc[j].w[i][0] = v[0]; rc[j].w[i][1] = v[1]; rc[j].w[i][2] = v[2]; rc[j].w[i][3] = v[3];
        } else {
          typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
          const u32x2_t* p = reinterpret_cast<const u32x2_t*>(cp);
          const u32x2_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1),
                        d = __builtin_nontemporal_load(p + 2);
          rc[j].w[i][0] = a[0]; rc[j].w[i][1] = a[1]; rc[j].w[i][2] = b[0]; rc[j].w[i][3] = b[1];
          rc[j].w[i][4] = d[0]; rc[j].w[i][5] = d[1];
        }
        rc[j].sc[i] = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>((j ? scales1 : scales0) + (size_t)ch * 8));
      }
    }
  }
}

// Masks and the bf16 2.0 pattern of the 2-bit decode, held in VGPRs so that each pair is one
// v_and_or_b32 (gfx9 VOP3 takes no literal operand).
struct Q2Consts {
  uint32_t m0, m1, m2, magic;
};
STRATA_DEVICE Q2Consts q2_consts() {
  Q2Consts k{0x00030003u, 0x000C000Cu, 0x00300030u, 0x40004000u};
  asm volatile("" : "+v"(k.m0), "+v"(k.m1), "+v"(k.m2), "+v"(k.magic));
  return k;
}

// 2-bit word -> 8 bf16 pairs (codes m, m + 8).
STRATA_DEVICE void q2_word_pairs(uint32_t w, const Q2Consts& k, uint32_t out[8]) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  out[0] = (w & k.m0) | k.magic;    // codes 0, 8:  2 + q/64
  out[1] = (w & k.m1) | k.magic;    // codes 1, 9:  2 + q/16
  out[2] = (w & k.m2) | k.magic;    // codes 2, 10: 2 + q/4
  out[3] = (w6 & k.m0) | k.magic;   // codes 3, 11
  out[4] = (w6 & k.m1) | k.magic;   // codes 4, 12
  out[5] = (w6 & k.m2) | k.magic;   // codes 5, 13
  out[6] = (w12 & k.m0) | k.magic;  // codes 6, 14
  out[7] = (w12 & k.m1) | k.magic;  // codes 7, 15
}

// 3-bit: 16 codes = 48 bits; bf16(4 + q/2) = 0x4080 | q << 4.
STRATA_DEVICE void q3_word_pairs(uint64_t v, uint32_t out[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t qa = (uint32_t)(v >> (3 * m)) & 7u;
    const uint32_t qb = (uint32_t)(v >> (3 * (m + 8))) & 7u;
    out[m] = (0x4080u | (qa << 4)) | ((0x4080u | (qb << 4)) << 16);
  }
}

// Word q (0..3) of a chunk (its code words cw) as bf16 pairs.
template <int FMT>
STRATA_DEVICE void chunk_word_pairs(const uint32_t* cw, int q, const Q2Consts& k, uint32_t pr[8]) {
  if constexpr (FMT == 2) {
    q2_word_pairs(cw[q], k, pr);
  } else {
    // block q/2 = words (q/2)*3 .. +2; word q%2 = bits 48*(q%2) .. of the block's 96 bits
    const int b = (q >> 1) * 3;
    const uint64_t lo = (uint64_t)cw[b] | ((uint64_t)cw[b + 1] << 32);
    const uint64_t v = (q & 1) ? ((lo >> 48) | ((uint64_t)cw[b + 2] << 16)) : lo;
    q3_word_pairs(v, pr);
  }
}

// Adds the 8 bf16 pair products of a word to two accumulation chains.
STRATA_DEVICE void dot8(const uint32_t pr[8], const uint32_t xw[8], float& p0, float& p1) {
#pragma unroll
  for (int m = 0; m < 8; m += 2) {
    p0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr[m]),
                                         __builtin_bit_cast(bf16x2_t, xw[m]), p0, false);
    p1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr[m + 1]),
                                         __builtin_bit_cast(bf16x2_t, xw[m + 1]), p1, false);
  }
}

// Partial dot products of NR weight rows (this lane's chunks) with one staged activation row;
// the activations are read from LDS once per word and applied to all NR rows.
template <int FMT, int MC, int NR>
STRATA_DEVICE void row_dots(RowChunks<FMT, MC> (&rc)[NR], int nchunk, int c0, int cstep,
                            const uint32_t* prow, const float* crow, float (&acc)[NR]) {
  const Q2Consts kq = q2_consts();
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int ch = c0 + cstep * i;
    if (ch < nchunk) {
      const float2 cc = *reinterpret_cast<const float2*>(crow + 2 * ch);
      float p[NR][2][2];  // [row][block][chain]
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        p[j][0][0] = -cc.x;
        p[j][1][0] = -cc.y;
        p[j][0][1] = 0.0f;
        p[j][1][1] = 0.0f;
        // Decode afresh for every activation row: an empty asm hides that the code words are the
        // same on each call, so the compiler does not keep all decoded pairs of the row live
        // across the caller's token loop (which would cost occupancy).
#pragma unroll
        for (int q = 0; q < RowChunks<FMT, MC>::kWords; ++q) asm volatile("" : "+v"(rc[j].w[i][q]));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(prow + kChunkDwords * ch + 8 * q);
        const u32x4_t x0 = xp[0], x1 = xp[1];
        const uint32_t xw[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          uint32_t pr[8];
          chunk_word_pairs<FMT>(rc[j].w[i], q, kq, pr);
          dot8(pr, xw, p[j][q >> 1][0], p[j][q >> 1][1]);
        }
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const float d0 = f16_to_f32((uint16_t)(rc[j].sc[i] & 0xFFFFu));
        const float d1 = f16_to_f32((uint16_t)(rc[j].sc[i] >> 16));
        acc[j] = __builtin_fmaf(d0, p[j][0][0] + p[j][0][1], acc[j]);
        acc[j] = __builtin_fmaf(d1, p[j][1][0] + p[j][1][1], acc[j]);
      }
    }
    // one chunk's activations at a time: keeps the register footprint at four waves per SIMD,
    // which hide the LDS latency better than hoisted loads would
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Contiguous range of K1's items (distinct expert d, block of rows) of this workgroup, balanced by
// work: an item's dot products are done once per token of its expert, so item (d, q) weighs
// dtp[d], and workgroup b takes the items whose weight prefix falls in [b W / G, (b + 1) W / G),
// W = blocks * S.  (With equal item counts, the workgroups holding an expert that two tokens
// picked took twice as long, and the slowest workgroup sets the kernel's end.)  Every wave finds
// its range with a scan across its lanes (two distinct experts a lane: nd <= 128), not a walk
// through the table.
STRATA_DEVICE void item_range(const RouteTable& rt, int blocks, int S, int& begin, int& end) {
  const int G = kGrid, b = blockIdx.x;  // the launch grid (a constant: no dispatch-packet read)
  const int lane = threadIdx.x & 63, nd = rt.nd;
  const int t0 = 2 * lane < nd ? rt.dtp[2 * lane] : 0;
  const int t1 = 2 * lane + 1 < nd ? rt.dtp[2 * lane + 1] : 0;
  const int inc = wave_scan_dpp(t0 + t1);  // tokens of the distinct experts 0 .. 2 lane + 1
  // the first item whose weight prefix is >= target (l is uniform: lane reads, no shuffles)
  auto item_at = [&](int target) {
    const uint64_t hit = __ballot(2 * lane < nd && inc * blocks >= target);
    if (hit == 0) return nd * blocks;
    const int l = __ffsll((unsigned long long)hit) - 1;
    const int ta = __builtin_amdgcn_readlane(t0, l), tb = __builtin_amdgcn_readlane(t1, l);
    const int ex = __builtin_amdgcn_readlane(inc, l) - ta - tb;
    const bool first = (ex + ta) * blocks >= target;
    const int d = first ? 2 * l : 2 * l + 1, cum = first ? ex : ex + ta, tp = first ? ta : tb;
    return d * blocks + (target - cum * blocks + tp - 1) / tp;
  };
  const int W = blocks * S;
  begin = item_at((b * W + G - 1) / G);
  end = item_at(((b + 1) * W + G - 1) / G);
}

// ---------------------------------------------------------------------------------------------
// K1: route + gate/up GEMV + SiLU*mul.  Items (distinct expert d, block of 4 rows of I), one wave
// each (16 lanes per row).
//
// RES (layer stacks): the input is the residual stream h (fp32) and x = bf16(h / rms(h)) is formed
// here.  While the routing waves route, every other thread loads its blocks of h (at most two:
// T * H / 32 <= 1024 blocks over >= 512 threads), keeps them in registers and leaves each block's
// sum of squares in LDS.  After the routing barrier a thread sums its token's block sums (in block
// order, four interleaved partial sums), scales and stages its blocks, and one more barrier
// publishes x.

// Dot product of 8 bf16 values of weights and activations (natural order), fp32 accumulation.
// (Named components: a subscripted vector element bit-cast inside an unrolled loop has compiled to
// element 0 every time.)
STRATA_DEVICE float bf16_dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, x), acc, false);
}
STRATA_DEVICE float bf16_dot8(const u32x4_t& w, const u32x4_t& x, float acc) {
  acc = bf16_dot2(w.x, x.x, acc);
  acc = bf16_dot2(w.y, x.y, acc);
  acc = bf16_dot2(w.z, x.z, acc);
  return bf16_dot2(w.w, x.w, acc);
}

// fp32 pair -> two bf16 (round to nearest even) in one word, low half first.
STRATA_DEVICE uint32_t bf16_pair(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <int FMT, int MC, bool RES>
__global__ __launch_bounds__(kUpThreads) void decode_up_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ h_res, float eps,
    const float* __restrict__ logits, int T, int E, int k, int H,
    int I, const uint8_t* __restrict__ gate_codes, const uint8_t* __restrict__ up_codes,
    const uint16_t* __restrict__ gate_scales, const uint16_t* __restrict__ up_scales,
    uint32_t* __restrict__ a_st /* [S][I/2] staged a, unpadded */, int* __restrict__ ids_ws,
    float* __restrict__ w_ws, GlobalTable* __restrict__ gt, const uint16_t* __restrict__ a_sh,
    const uint16_t* __restrict__ w_sd, int Is, float* __restrict__ y_sh, int sh_acc) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ RouteTable rt;
  __shared__ __align__(16) float part[RES ? kDecMaxT * 128 : 4];  // block sums of squares of h
  __shared__ __align__(16) uint64_t sel[kDecMaxT][80];  // the routing waves' selection LDS
  const int tid = threadIdx.x, S = T * k;
  const int nb = H / 32, nblk = T * nb, nchunk = H / 64, rs = kChunkDwords * nchunk;
  uint32_t* pairs = reinterpret_cast<uint32_t*>(smem);
  float* cs = reinterpret_cast<float*>(smem + (size_t)T * rs * 4);
  int* scratch = reinterpret_cast<int*>(smem + (size_t)T * staged_row_bytes(H));
  table_clear<kUpThreads>(rt, S, E, scratch);  // visible after the barrier below
  // waves 0 .. T-1 route one token each while the other waves stage x
  const int nr = T * 64;
  f32x4_t hv[RES ? 2 : 1][8];  // RES: this thread's blocks of h (blocks tid - nr + j (1024 - nr))
  if (tid < nr) {
    route_token(logits, tid >> 6, E, k, rt.ids, rt.w, sel[tid >> 6]);
  } else if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int b = tid - nr + j * (kUpThreads - nr);
      if (b < nblk) {
        const int t = b / nb, blk = b - t * nb;
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(h_res + (size_t)t * H + blk * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[j][i] = src[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int b = tid - nr + j * (kUpThreads - nr);
      if (b < nblk) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) ss = __builtin_fmaf(hv[j][i][q], hv[j][i][q], ss);
        part[b] = ss;
      }
    }
  } else {
    for (int b = tid - nr; b < nblk; b += kUpThreads - nr) {
      u32x4_t v[4];
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)b * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = src[i];
      stage_block<FMT>(v, pairs + (b / nb) * rs, cs + (b / nb) * nb, b % nb);
    }
  }
  // Block calls: the shared expert's down projection for rows [b R, (b + 1) R) of H (R = H / 256),
  // y[t][row] (=|+=) sum_n W_sd[row][n] a_sh[t][n], by the waves that staged x, while the routing
  // waves are still routing (they would otherwise wait at the barrier).  K2 then accumulates.
  if constexpr (!RES) {
    if (a_sh != nullptr && tid >= nr) {
      const int nsw = (kUpThreads - nr) >> 6, sw = (tid - nr) >> 6, sl = tid & 63;
      const int R = H / kGrid, h0 = blockIdx.x * R, np = Is >> 3;  // 16-byte pieces per row
      const u32x4_t* av = reinterpret_cast<const u32x4_t*>(a_sh);
      for (int r = sw; r < R; r += nsw) {
        const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(w_sd + (size_t)(h0 + r) * Is);
        float acc[kDecMaxT];
#pragma unroll
        for (int t = 0; t < kDecMaxT; ++t) acc[t] = 0.0f;
        for (int q0 = sl; q0 < np; q0 += 128) {
          const int q1 = q0 + 64;
          const u32x4_t z = {0u, 0u, 0u, 0u};
          const u32x4_t w0 = wrow[q0], w1 = q1 < np ? wrow[q1] : z;
          u32x4_t x0[kDecMaxT], x1[kDecMaxT];
#pragma unroll
          for (int t = 0; t < kDecMaxT; ++t) {
            x0[t] = t < T ? av[(size_t)t * np + q0] : z;
            x1[t] = t < T && q1 < np ? av[(size_t)t * np + q1] : z;
          }
#pragma unroll
          for (int t = 0; t < kDecMaxT; ++t) {
            acc[t] = bf16_dot8(w0, x0[t], acc[t]);
            acc[t] = bf16_dot8(w1, x1[t], acc[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < kDecMaxT; ++t) {
          if (t < T) {
            const float v = wave_sum(acc[t]);
            if (sl == 0) {
              float* dst = y_sh + (size_t)t * H + h0 + r;
              *dst = sh_acc ? *dst + v : v;
            }
          }
        }
      }
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < S) { ids_ws[tid] = rt.ids[tid]; w_ws[tid] = rt.w[tid]; }
  build_table(rt, T, k, scratch);
  if (blockIdx.x == 0) {  // the table for K2
    if (tid == 0) gt->nd = rt.nd;
    if (tid < rt.nd) {
      gt->dexp[tid] = rt.dexp[tid];
      gt->dtp[tid] = rt.dtp[tid];
      *reinterpret_cast<uint2*>(gt->dslot[tid]) = *reinterpret_cast<const uint2*>(rt.dslot[tid]);
    }
  }
  const int blocks = I / kUpRows;
  int it, end;
  item_range(rt, blocks, S, it, end);
  if (it >= end) return;
  constexpr int CB = FMT == 2 ? 8 : 12;
  constexpr int kGroups = kUpThreads / 64;  // one wave per item
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, rl = lane >> 4;
  // (gate row, up row) of one item in flight per wave: a second batch of loads would only queue
  // behind the first (the load pipeline is already full), and costs registers
  constexpr bool kTwo = false;
  RowChunks<FMT, MC> gu[kTwo ? 2 : 1][2];
  auto load_item = [&](int item, RowChunks<FMT, MC> (&rr)[2]) {
    const int d = item / blocks, n = (item % blocks) * kUpRows + rl;
    const size_t row = (size_t)rt.dexp[d] * I + n;
    load_row_chunks<FMT, MC>(rr[0], tiled_row_codes<FMT>(gate_codes, row, nchunk),
                             tiled_row_scales(gate_scales, row, nchunk), nchunk, c, 16);
    load_row_chunks<FMT, MC>(rr[1], tiled_row_codes<FMT>(up_codes, row, nchunk),
                             tiled_row_scales(up_scales, row, nchunk), nchunk, c, 16);
  };
  // a = SiLU(g) u, rounded to bf16, goes out already in K2's staged layout without the chunk
  // padding: row n = 16 q + rsub is value rsub of word q & 3 of chunk q >> 2, i.e. half rsub >> 3
  // of pair m = rsub & 7, multiplied by that pair's power of two (exact).
  auto compute_item = [&](int item, RowChunks<FMT, MC> (&rr)[2]) {
    const int d = item / blocks, n = (item % blocks) * kUpRows + rl;
    const int q = n >> 4, rsub = n & 15, m_a = rsub & 7;
    const float sc_a = FMT == 2 ? (m_a % 3 == 0 ? 64.0f : m_a % 3 == 1 ? 16.0f : 4.0f) : 2.0f;
    const int Tp = rt.dtp[d];
    for (int tt = 0; tt < Tp; ++tt) {
      const int t = rt.dtok[d][tt];
      float acc[2];
      row_dots<FMT, MC, 2>(rr, nchunk, c, 16, pairs + t * rs, cs + t * nb, acc);
      const float gs = sum16(acc[0]), us = sum16(acc[1]);
      const int slot = rt.dslot[d][tt];
      const float a = gs / (1.0f + expf(-gs)) * us;
      const float xa = __uint_as_float((uint32_t)f32_to_bf16(a) << 16);
      if (c == 0) {
        uint32_t* word = a_st + (size_t)slot * (I / 2) + 32 * (q >> 2) + 8 * (q & 3) + m_a;
        reinterpret_cast<uint16_t*>(word)[rsub >> 3] = (uint16_t)(__float_as_uint(xa * sc_a) >> 16);
      }
    }
  };
  // RES: stage x = bf16(h / rms) from registers while the first weights load; where the held
  // blocks and one item's weight registers do not fit together (Q3 with >= 3 chunks per lane, Q2
  // with 4) the blocks are staged before the first loads instead.
  constexpr bool kStageEarly = FMT == 3 ? MC >= 3 : MC >= 4;
  auto stage_res = [&]() {
    if (tid >= nr) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int b = tid - nr + j * (kUpThreads - nr);
        if (b < nblk) {
          const int t = b / nb, blk = b - t * nb;
          const f32x4_t* pt = reinterpret_cast<const f32x4_t*>(part + t * nb);
          f32x4_t acc = pt[0];
          for (int q = 1; q < nb / 4; ++q) acc += pt[q];
          const float ss = (acc[0] + acc[1]) + (acc[2] + acc[3]);
          const float inv = 1.0f / sqrtf(ss / (float)H + eps);
          u32x4_t v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4_t p = hv[j][2 * i], q = hv[j][2 * i + 1];
            v[i] = u32x4_t{bf16_pair(p[0] * inv, p[1] * inv), bf16_pair(p[2] * inv, p[3] * inv),
                           bf16_pair(q[0] * inv, q[1] * inv), bf16_pair(q[2] * inv, q[3] * inv)};
          }
          stage_block<FMT>(v, pairs + t * rs, cs + t * nb, blk);
        }
      }
    }
    __syncthreads();
  };
  if constexpr (RES && kStageEarly) stage_res();
  // (no barrier after the first weight loads: they are accepted only as fast as data returns, so
  // a barrier would hold every wave until the whole first batch had been issued)
  it += wave;
  if (it < end) load_item(it, gu[0]);
  if constexpr (RES && !kStageEarly) stage_res();
  if constexpr (kTwo) {
    if (it + kGroups < end) load_item(it + kGroups, gu[kTwo ? 1 : 0]);
    for (; it < end; it += 2 * kGroups) {
      compute_item(it, gu[0]);
      if (it + 2 * kGroups < end) load_item(it + 2 * kGroups, gu[0]);
      if (it + kGroups >= end) break;
      compute_item(it + kGroups, gu[kTwo ? 1 : 0]);
      if (it + 3 * kGroups < end) load_item(it + 3 * kGroups, gu[kTwo ? 1 : 0]);
    }
  } else {
    for (; it < end; it += kGroups) {
      compute_item(it, gu[0]);
      if (it + kGroups < end) load_item(it + kGroups, gu[0]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// K2: down GEMV + combine.  Workgroup b owns rows [b R, (b+1) R) of H for every distinct expert;
// units (distinct expert d, row r), LPU lanes per unit.

template <int FMT, int MC, int LPU>
__global__ __launch_bounds__(kDnThreads) void decode_down_kernel(
    const uint32_t* __restrict__ a_st, const GlobalTable* __restrict__ gt,
    const float* __restrict__ w_ws,
    int T, int E, int k, int H, int I, const uint8_t* __restrict__ down_codes,
    const uint16_t* __restrict__ down_scales, float* __restrict__ y, int accumulate) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ RouteTable rt;
  __shared__ float outs[kDecMaxS * kDecMaxR];  // [slot][r]
  const int tid = threadIdx.x, S = T * k;
  const int R = H / kGrid, h0 = blockIdx.x * R;
  const int nb = I / 32, nchunk = I / 64, rs = kChunkDwords * nchunk;
  uint32_t* pairs = reinterpret_cast<uint32_t*>(smem);
  float* cs = reinterpret_cast<float*>(smem + (size_t)S * rs * 4);
  // Every thread loads its 16-byte pieces of the slots' staged a (K1 wrote it in the layout
  // below, without the chunk padding), while waves 8-15 also fetch the routing table.  After the
  // barrier each wave writes its pieces to LDS and the block constants C = sum coef x (a block is
  // four consecutive pieces, so four consecutive lanes: a quad sum), counts itself in an LDS
  // counter and starts its weight loads; the counter (not a barrier, which would hold everyone
  // behind the throttled weight loads) tells the waves when the staged a is complete.
  constexpr int kStage = 512;
  __shared__ int staged_waves;
  const int ppr = I / 8, ncp = S * ppr;  // pieces per row; pieces
  const u32x4_t* src_st = reinterpret_cast<const u32x4_t*>(a_st);
  u32x4_t cv[kDnPieces];
#pragma unroll
  for (int i = 0; i < kDnPieces; ++i)
    if (tid + kDnThreads * i < ncp) cv[i] = src_st[tid + kDnThreads * i];
  if (tid >= kStage) {
    const int q = tid - kStage;
    if (q == 0) { rt.nd = gt->nd; staged_waves = 0; }
    if (q < S) {
      rt.w[q] = w_ws[q];
      rt.dexp[q] = gt->dexp[q];
      rt.dtp[q] = gt->dtp[q];
      *reinterpret_cast<uint2*>(rt.dslot[q]) = *reinterpret_cast<const uint2*>(gt->dslot[q]);
    }
  }
  __syncthreads();
  constexpr int CB = FMT == 2 ? 8 : 12;
  constexpr int kGroups = kDnThreads / LPU;
  // units (distinct expert d, row pair r < RH): rows r and r + RH (the second repeats r when it
  // falls outside the R rows), so that each activation read from LDS serves two rows
  const int RH = (R + 1) / 2, U = rt.nd * RH, g = tid / LPU, j = tid % LPU;
  // Two units' weights in flight per lane group, except where two do not fit in the registers
  // beside everything else (3-bit with >= 3 chunks per lane, 2-bit with 4): one unit at a time
  // there (with 256 lane groups and 6 units per distinct expert a group rarely has a second).
  constexpr bool kTwoUnits = FMT == 3 ? MC < 3 : MC < 4;
  RowChunks<FMT, MC> wr[kTwoUnits ? 2 : 1][2];
  auto unit_rows = [&](int u, int& r0, int& r1) {
    r0 = u % RH;
    r1 = r0 + RH < R ? r0 + RH : r0;
  };
  auto load_unit = [&](int u, RowChunks<FMT, MC> (&rr)[2]) {
    int r0, r1;
    unit_rows(u, r0, r1);
    const size_t base = (size_t)rt.dexp[u / RH] * H + h0;
    load_row_pair_chunks<FMT, MC>(rr, tiled_row_codes<FMT>(down_codes, base + r0, nchunk),
                                  tiled_row_scales(down_scales, base + r0, nchunk),
                                  tiled_row_codes<FMT>(down_codes, base + r1, nchunk),
                                  tiled_row_scales(down_scales, base + r1, nchunk), nchunk, j, LPU);
  };
  {
    // piece q: row q / ppr, chunk (q % ppr) / 8, dwords 4 (q % 8) .. + 3 of the chunk, pairs
    // m = 4 (q % 2) .. + 3 of its word; the stored values are x * s(m), so coef(m) x is
    // (coef(m) / s(m)) times them, exactly
    const int m0 = 4 * (tid & 1);
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + e;
      f[e] = FMT == 2 ? (m % 3 == 0 ? 2.0f + 1.5f / 64.0f : m % 3 == 1 ? 2.0f + 1.5f / 16.0f
                                                                     : 2.0f + 1.5f / 4.0f)
                      : 11.5f / 2.0f;
    }
    // (row, position) of piece q, stepped from piece to piece instead of divided out each time
    const int rstep = kDnThreads / ppr, pstep = kDnThreads - rstep * ppr;
    int row = tid / ppr, pr = tid - row * ppr;
#pragma unroll
    for (int i = 0; i < kDnPieces; ++i) {
      const int q = tid + kDnThreads * i;
      if (q - (q & 3) < ncp) {  // the whole quad is in range or out (ncp is a multiple of 4)
        *reinterpret_cast<u32x4_t*>(pairs + row * rs + kChunkDwords * (pr >> 3) + 4 * (pr & 7)) = cv[i];
        float c = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c = __builtin_fmaf(f[e], __uint_as_float(cv[i][e] << 16), c);
          c = __builtin_fmaf(f[e], __uint_as_float(cv[i][e] & 0xFFFF0000u), c);
        }
        c = sum4(c);
        if ((q & 3) == 0) cs[q >> 2] = c;
      }
      row += rstep;
      pr += pstep;
      if (pr >= ppr) {
        pr -= ppr;
        ++row;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if ((tid & 63) == 0) atomicAdd(&staged_waves, 1);
  }
  if (g < U) load_unit(g, wr[0]);
  if constexpr (kTwoUnits)
    if (g + kGroups < U) load_unit(g + kGroups, wr[kTwoUnits ? 1 : 0]);
  while (__hip_atomic_load(&staged_waves, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kDnThreads / 64)
    __builtin_amdgcn_s_sleep(1);
  auto compute_unit = [&](int u, RowChunks<FMT, MC> (&rr)[2]) {
    const int d = u / RH;
    int r0, r1;
    unit_rows(u, r0, r1);
    const int Tp = rt.dtp[d];  // uniform over the unit's lanes
    for (int tt = 0; tt < Tp; ++tt) {
      const int slot = rt.dslot[d][tt];
      float acc[2];
      row_dots<FMT, MC, 2>(rr, nchunk, j, LPU, pairs + slot * rs, cs + slot * nb, acc);
      const float v0 = LPU == 4 ? sum4(acc[0]) : sum16(acc[0]);
      const float v1 = LPU == 4 ? sum4(acc[1]) : sum16(acc[1]);
      if (j == 0) {
        outs[slot * R + r0] = v0;
        outs[slot * R + r1] = v1;  // r1 == r0 rewrites the same value
      }
    }
  };
  if constexpr (kTwoUnits) {
    for (int u = g; u < U; u += 2 * kGroups) {
      compute_unit(u, wr[0]);
      if (u + 2 * kGroups < U) load_unit(u + 2 * kGroups, wr[0]);
      if (u + kGroups < U) {
        compute_unit(u + kGroups, wr[kTwoUnits ? 1 : 0]);
        if (u + 3 * kGroups < U) load_unit(u + 3 * kGroups, wr[kTwoUnits ? 1 : 0]);
      }
    }
  } else {
    for (int u = g; u < U; u += kGroups) {
      compute_unit(u, wr[0]);
      if (u + kGroups < U) load_unit(u + kGroups, wr[0]);
    }
  }
  __syncthreads();
  for (int o = tid; o < T * R; o += kDnThreads) {
    const int t = o / R, r = o % R;
    float acc = 0.0f;
    for (int jj = 0; jj < k; ++jj) acc = __builtin_fmaf(rt.w[t * k + jj], outs[(t * k + jj) * R + r], acc);
    float* dst = y + (size_t)t * H + h0 + r;
    *dst = accumulate ? *dst + acc : acc;
  }
}

// ---------------------------------------------------------------------------------------------
// Host side

static size_t up_lds_bytes(int T, int E, int H) {
  return (size_t)T * staged_row_bytes(H) + (size_t)E * 4;
}
static size_t dn_lds_bytes(int T, int E, int k, int I) {
  const size_t st = (size_t)T * k * staged_row_bytes(I), sc = (size_t)E * 4;
  return st > sc ? st : sc;
}
constexpr size_t kDecLdsLimit = 160 * 1024 - 16 * 1024;  // dynamic LDS beside the static tables

bool decode_fits(int T, int E, int k, int H, int I) {
  if (T < 1 || T > kDecMaxT || T * k > kDecMaxS || E > 1024) return false;
  if (H % 256 || H > 4096 || I % 128 || I > 4096) return false;
  // (K2 holds every slot's staged a in registers on its way to LDS: <= kDnPieces pieces a thread)
  const size_t pieces = (size_t)T * k * I / 8;
  return up_lds_bytes(T, E, H) <= kDecLdsLimit && dn_lds_bytes(T, E, k, I) <= kDecLdsLimit &&
         pieces <= (size_t)kDnPieces * kDnThreads;
}

// Workspace: ids [S] int32 | w [S] fp32 | routing table | staged a [S][I/2] (K2's LDS layout
// without the chunk padding)
size_t decode_workspace_bytes(int T, int E, int k, int H, int I) {
  (void)E; (void)H;
  const size_t S = (size_t)T * k;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return up(S * 4) + up(S * 4) + up(sizeof(GlobalTable)) + up(S * I * 2);
}

template <typename K>
static void allow_lds(K kernel) {
  hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecLdsLimit);
}

template <int F>
static void allow_all_decode_lds() {
  allow_lds(decode_up_kernel<F, 1, false>); allow_lds(decode_up_kernel<F, 2, false>);
  allow_lds(decode_up_kernel<F, 3, false>); allow_lds(decode_up_kernel<F, 4, false>);
  allow_lds(decode_up_kernel<F, 1, true>); allow_lds(decode_up_kernel<F, 2, true>);
  allow_lds(decode_up_kernel<F, 3, true>); allow_lds(decode_up_kernel<F, 4, true>);
  allow_lds(decode_down_kernel<F, 1, 4>); allow_lds(decode_down_kernel<F, 2, 4>);
  allow_lds(decode_down_kernel<F, 3, 4>); allow_lds(decode_down_kernel<F, 4, 4>);
  allow_lds(decode_down_kernel<F, 2, 16>); allow_lds(decode_down_kernel<F, 3, 16>);
  allow_lds(decode_down_kernel<F, 4, 16>);
}

hipError_t launch_decode(int fmt, const uint16_t* x, const float* h_res, float eps,
                         const float* logits, int T, int E, int k,
                         int H, int I, const void* gate_codes, const void* up_codes,
                         const void* down_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, const uint16_t* down_scales, float* y,
                         int accumulate, int* ids_out, float* w_out, void* ws, hipStream_t s,
                         const uint16_t* a_sh, const uint16_t* w_sd, int Is) {
  if (!decode_fits(T, E, k, H, I)) return hipErrorInvalidValue;
  if (a_sh && (h_res || Is < 8 || Is % 8)) return hipErrorInvalidValue;
  const int sh_acc = accumulate, acc_dn = a_sh ? 1 : accumulate;
  static std::once_flag once;
  std::call_once(once, [] { allow_all_decode_lds<2>(); allow_all_decode_lds<3>(); });
  const size_t S = (size_t)T * k;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  int* ids = ids_out ? ids_out : reinterpret_cast<int*>(p);
  p += up(S * 4);
  float* w = w_out ? w_out : reinterpret_cast<float*>(p);
  p += up(S * 4);
  GlobalTable* gt = reinterpret_cast<GlobalTable*>(p);
  p += up(sizeof(GlobalTable));
  uint32_t* a_st = reinterpret_cast<uint32_t*>(p);
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  const size_t lds_up = up_lds_bytes(T, E, H), lds_dn = dn_lds_bytes(T, E, k, I);
  const int mc_up = (H / 64 + 15) / 16;                 // 1..4 chunks per lane (16 lanes per row)
  const int nch_dn = I / 64;
  const int lpu = nch_dn <= 16 ? 4 : 16;                 // lanes per down row
  const int mc_dn = (nch_dn + lpu - 1) / lpu;            // 1..4
#define STRATA_UP(F, M)                                                                          \
  do {                                                                                           \
    if (h_res)                                                                                   \
      decode_up_kernel<F, M, true><<<kGrid, kUpThreads, lds_up, s>>>(                            \
          x, h_res, eps, logits, T, E, k, H, I, gc, uc, gate_scales, up_scales, a_st, ids, w, gt, a_sh, w_sd, Is, y, sh_acc); \
    else                                                                                         \
      decode_up_kernel<F, M, false><<<kGrid, kUpThreads, lds_up, s>>>(                           \
          x, h_res, eps, logits, T, E, k, H, I, gc, uc, gate_scales, up_scales, a_st, ids, w, gt, a_sh, w_sd, Is, y, sh_acc); \
  } while (0)
#define STRATA_DN(F, M, L)                                                                       \
  decode_down_kernel<F, M, L><<<kGrid, kDnThreads, lds_dn, s>>>(a_st, gt, w, T, E, k, H, I, \
                                                                   dc, down_scales, y, acc_dn)
#define STRATA_DEC(F)                                                                            \
  switch (mc_up) { case 1: STRATA_UP(F, 1); break; case 2: STRATA_UP(F, 2); break;              \
                   case 3: STRATA_UP(F, 3); break; default: STRATA_UP(F, 4); break; }           \
  if (lpu == 4) {                                                                                \
    switch (mc_dn) { case 1: STRATA_DN(F, 1, 4); break; case 2: STRATA_DN(F, 2, 4); break;       \
                     case 3: STRATA_DN(F, 3, 4); break; default: STRATA_DN(F, 4, 4); break; }    \
  } else {                                                                                       \
    switch (mc_dn) { case 2: STRATA_DN(F, 2, 16); break; case 3: STRATA_DN(F, 3, 16); break;     \
                     default: STRATA_DN(F, 4, 16); break; }                                      \
  }
  if (fmt == 2) {
    STRATA_DEC(2)
  } else {
    STRATA_DEC(3)
  }
#undef STRATA_UP
#undef STRATA_DN
#undef STRATA_DEC
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Fixed scratch for callers that cannot allocate (strata_moe_decode_static): the decode path's
// workspace in a device array of this library, one per GPU, reused by every such call on it.

// (every shape within the decode limits fits: the largest workspace they allow is 126,720 bytes)
constexpr size_t kDecStaticScratch = 128 * 1024;
static __device__ __align__(256) uint8_t scratch[kDecStaticScratch];

size_t decode_static_scratch_bytes() { return kDecStaticScratch; }

// The current device's address of `scratch`, looked up once per device (hipGetSymbolAddress with
// that device current) and kept; host code never uses the array's name as an address.
hipError_t decode_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace strata
