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
//  K1 up:   every workgroup routes all T tokens itself (one wave per token), lists the distinct
//           experts and the (token, slot) pairs of each, and works through a contiguous range of
//           items (distinct expert, 16 rows of I): a = SiLU(g) * u per token, rounded to bf16.
//           Workgroup 0 publishes the routing for K2 and the caller.
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

namespace strata {

constexpr int kDecThreads = 256;   // K1: 4 waves
constexpr int kDnThreads = 1024;   // K2: 16 waves, one workgroup per CU
constexpr int kDnGrid = 256;
constexpr int kDecMaxT = 8;
constexpr int kDecMaxS = 128;      // T * k <= 8 * 16
constexpr int kDecMaxR = 16;       // rows of H per K2 workgroup (H <= 4096)
constexpr int kUpRows = 16;        // rows of I per K1 item (4 per wave, 16 lanes per row)

// ---------------------------------------------------------------------------------------------
// DPP wave reductions

template <int CTRL, int ROW_MASK = 0xF>
STRATA_DEVICE int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
STRATA_DEVICE float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

// Sum over each group of 16 lanes (every lane of the group receives it).
STRATA_DEVICE float sum16(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return v;
}
// Sum over each group of 4 lanes.
STRATA_DEVICE float sum4(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  return v;
}

// Wave-wide max of unsigned keys / min of ints, result uniform (read from lane 63).
STRATA_DEVICE uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<0xB1>((int)v));
  v = max(v, (uint32_t)dpp_i<0x4E>((int)v));
  v = max(v, (uint32_t)dpp_i<0x124>((int)v));
  v = max(v, (uint32_t)dpp_i<0x128>((int)v));
  v = max(v, (uint32_t)dpp_i<0x142, 0xA>((int)v));  // row_bcast:15
  v = max(v, (uint32_t)dpp_i<0x143, 0xC>((int)v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
STRATA_DEVICE int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x124>(v));
  v = min(v, dpp_i<0x128>(v));
  v = min(v, dpp_i<0x142, 0xA>(v));
  v = min(v, dpp_i<0x143, 0xC>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Order-preserving map of a logit to an unsigned key (-0 is first made +0, so equal logits get
// equal keys), and back.
STRATA_DEVICE uint32_t route_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
STRATA_DEVICE float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Top-k of one token's logits by one wave: k rounds of "largest remaining logit, equal logits to
// the lower expert index"; weights = softmax over the k kept logits (same rule as the router).
template <int NPL>
STRATA_DEVICE void route_token_wave(const float* __restrict__ row, int E, int k, int* ids_out,
                                    float* w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(row[e]) : 0u;
    if (e >= E) taken |= 1u << i;
  }
  uint32_t my_key = 0;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t bk = 0;
    int bi = -1;  // this lane's best remaining entry (lowest i among equal keys)
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (!((taken >> i) & 1u) && (bi < 0 || key[i] > bk)) { bk = key[i]; bi = i; }
    const uint32_t m = wave_max_u32(bi >= 0 ? bk : 0u);
    const bool cand = bi >= 0 && bk == m;
    const uint64_t ball = __ballot(cand);
    int win;
    if (__popcll(ball) == 1) {  // the usual case: one lane holds the maximum
      const int wl = __ffsll((unsigned long long)ball) - 1;
      win = wl + 64 * __builtin_amdgcn_readlane(bi, wl);
    } else {                    // equal logits in several lanes: lowest expert index
      win = wave_min_i(cand ? lane + 64 * bi : 0x7FFFFFFF);
    }
    if ((win & 63) == lane) taken |= 1u << (win >> 6);
    if (lane == j) { my_key = m; my_i = win; }
  }
  const float top = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
  const float ex = lane < k ? expf(key_value(my_key) - top) : 0.0f;
  const float den = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_i;
    w_out[lane] = ex / den;
  }
}

STRATA_DEVICE void route_all_tokens(const float* __restrict__ logits, int T, int E, int k,
                                    int* ids_s, float* w_s) {
  const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  for (int t = wave; t < T; t += nwaves) {
    const float* row = logits + (size_t)t * E;
    if (E <= 64) route_token_wave<1>(row, E, k, ids_s + t * k, w_s + t * k);
    else if (E <= 128) route_token_wave<2>(row, E, k, ids_s + t * k, w_s + t * k);
    else if (E <= 256) route_token_wave<4>(row, E, k, ids_s + t * k, w_s + t * k);
    else if (E <= 512) route_token_wave<8>(row, E, k, ids_s + t * k, w_s + t * k);
    else route_token_wave<16>(row, E, k, ids_s + t * k, w_s + t * k);
  }
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

// Builds the table from rt.ids (visible to the workgroup).  scratch: 2 E ints of LDS.
STRATA_DEVICE void build_table(RouteTable& rt, int T, int k, int E, int* scratch) {
  int* first_slot = scratch;      // per expert: lowest slot that picked it
  int* pos_of = scratch + E;      // per expert: its index in the distinct list
  __shared__ int wave_cnt[kDecMaxS / 64];
  const int S = T * k, q = threadIdx.x;
  for (int e = q; e < E; e += blockDim.x) first_slot[e] = 0x7FFFFFFF;
  if (q < S) rt.dtp[q] = 0;
  __syncthreads();
  if (q < S) atomicMin(&first_slot[rt.ids[q]], q);
  __syncthreads();
  const bool first = q < S && first_slot[rt.ids[q]] == q;
  const uint64_t ball = __ballot(first);
  const int lane = q & 63, wv = q >> 6;
  if (lane == 0 && wv < kDecMaxS / 64) wave_cnt[wv] = __popcll(ball);
  __syncthreads();
  if (first) {
    int pos = __popcll(ball & ((1ull << lane) - 1ull));
    for (int i = 0; i < wv; ++i) pos += wave_cnt[i];
    rt.dexp[pos] = rt.ids[q];
    pos_of[rt.ids[q]] = pos;
  }
  if (q == 0) rt.nd = wave_cnt[0] + (S > 64 ? wave_cnt[1] : 0);
  __syncthreads();
  // each slot appends itself to its expert's list; a token picks an expert at most once and the
  // per-token arithmetic does not depend on the position in the list
  if (q < S) {
    const int p = pos_of[rt.ids[q]];
    const int idx = atomicAdd(&rt.dtp[p], 1);
    rt.dtok[p][idx] = (uint8_t)(q / k);
    rt.dslot[p][idx] = (uint8_t)q;
  }
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

inline size_t staged_row_bytes(int K) { return (size_t)(K / 64) * kChunkDwords * 4 + (size_t)(K / 32) * 4; }

// ---------------------------------------------------------------------------------------------
// Weight rows: a lane holds chunks c0, c0 + cstep, ... (< nchunk) of a packed row, at most MC.

template <int FMT, int MC>
struct RowChunks {
  static constexpr int kWords = FMT == 2 ? 4 : 6;  // 32-bit words of code bytes per chunk
  uint32_t w[MC][kWords];
  uint32_t sc[MC];                                 // the chunk's two fp16 block scales
};

template <int FMT, int MC>
STRATA_DEVICE void load_row_chunks(RowChunks<FMT, MC>& rc, const uint8_t* row_codes,
                                   const uint16_t* row_scales, int nchunk, int c0, int cstep) {
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int ch = c0 + cstep * i;
    if (ch < nchunk) {
      if constexpr (FMT == 2) {
        const u32x4_t v = reinterpret_cast<const u32x4_t*>(row_codes)[ch];
        rc.w[i][0] = v[0]; rc.w[i][1] = v[1]; rc.w[i][2] = v[2]; rc.w[i][3] = v[3];
      } else {
        const uint2* p = reinterpret_cast<const uint2*>(row_codes + (size_t)ch * 24);
        const uint2 a = p[0], b = p[1], d = p[2];
        rc.w[i][0] = a.x; rc.w[i][1] = a.y; rc.w[i][2] = b.x; rc.w[i][3] = b.y;
        rc.w[i][4] = d.x; rc.w[i][5] = d.y;
      }
      rc.sc[i] = reinterpret_cast<const uint32_t*>(row_scales)[ch];
    }
  }
}

// 2-bit word -> 8 bf16 pairs (codes m, m + 8); magic = 0x40004000 (kept in a register).
STRATA_DEVICE void q2_word_pairs(uint32_t w, uint32_t magic, uint32_t out[8]) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  out[0] = (w & 0x00030003u) | magic;    // codes 0, 8:  2 + q/64
  out[1] = (w & 0x000C000Cu) | magic;    // codes 1, 9:  2 + q/16
  out[2] = (w & 0x00300030u) | magic;    // codes 2, 10: 2 + q/4
  out[3] = (w6 & 0x00030003u) | magic;   // codes 3, 11
  out[4] = (w6 & 0x000C000Cu) | magic;   // codes 4, 12
  out[5] = (w6 & 0x00300030u) | magic;   // codes 5, 13
  out[6] = (w12 & 0x00030003u) | magic;  // codes 6, 14
  out[7] = (w12 & 0x000C000Cu) | magic;  // codes 7, 15
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
STRATA_DEVICE void chunk_word_pairs(const uint32_t* cw, int q, uint32_t magic, uint32_t pr[8]) {
  if constexpr (FMT == 2) {
    q2_word_pairs(cw[q], magic, pr);
  } else {
    // block q/2 = words (q/2)*3 .. +2; word q%2 = bits 48*(q%2) .. of the block's 96 bits
    const int b = (q >> 1) * 3;
    const uint64_t lo = (uint64_t)cw[b] | ((uint64_t)cw[b + 1] << 32);
    const uint64_t v = (q & 1) ? ((lo >> 48) | ((uint64_t)cw[b + 2] << 16)) : lo;
    q3_word_pairs(v, pr);
  }
}

// init + sum of 8 bf16 pair products, two chains.
STRATA_DEVICE float dot8(const uint32_t pr[8], const uint32_t xw[8], float init) {
  float p0 = init, p1 = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; m += 2) {
    p0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr[m]),
                                         __builtin_bit_cast(bf16x2_t, xw[m]), p0, false);
    p1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr[m + 1]),
                                         __builtin_bit_cast(bf16x2_t, xw[m + 1]), p1, false);
  }
  return p0 + p1;
}

// Partial dot products of NR weight rows (this lane's chunks) with one staged activation row;
// the activations are read from LDS once per word and applied to all NR rows.
template <int FMT, int MC, int NR>
STRATA_DEVICE void row_dots(const RowChunks<FMT, MC> (&rc)[NR], int nchunk, int c0, int cstep,
                            const uint32_t* prow, const float* crow, float (&acc)[NR]) {
  // bf16 2.0 in both halves, opaque to constant folding so that it lives in a VGPR
  const uint32_t magic = 0x40004000u | (uint32_t)(threadIdx.x >> 10);
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int ch = c0 + cstep * i;
    if (ch < nchunk) {
      const float2 cc = *reinterpret_cast<const float2*>(crow + 2 * ch);
      float p[NR][2];
      uint32_t cw[NR][RowChunks<FMT, MC>::kWords];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        p[j][0] = -cc.x;
        p[j][1] = -cc.y;
        // Decode afresh for every activation row: an empty asm hides that the code words are the
        // same on each call, so the compiler does not keep all decoded pairs of the row live
        // across the caller's token loop (which would cost occupancy).
#pragma unroll
        for (int q = 0; q < RowChunks<FMT, MC>::kWords; ++q) {
          cw[j][q] = rc[j].w[i][q];
          asm volatile("" : "+v"(cw[j][q]));
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(prow + kChunkDwords * ch + 8 * q);
        const u32x4_t x0 = xp[0], x1 = xp[1];
        const uint32_t xw[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          uint32_t pr[8];
          chunk_word_pairs<FMT>(cw[j], q, magic, pr);
          p[j][q >> 1] = dot8(pr, xw, p[j][q >> 1]);
        }
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const float d0 = f16_to_f32((uint16_t)(rc[j].sc[i] & 0xFFFFu));
        const float d1 = f16_to_f32((uint16_t)(rc[j].sc[i] >> 16));
        acc[j] = __builtin_fmaf(d0, p[j][0], acc[j]);
        acc[j] = __builtin_fmaf(d1, p[j][1], acc[j]);
      }
    }
    // one chunk's activations at a time: keeps the register footprint at four waves per SIMD,
    // which hide the LDS latency better than hoisted loads would
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Contiguous range of work items of this workgroup.
STRATA_DEVICE void item_range(int n_items, int& begin, int& end) {
  const int G = gridDim.x, b = blockIdx.x;
  const int per = n_items / G, extra = n_items % G;
  begin = b * per + (b < extra ? b : extra);
  end = begin + per + (b < extra ? 1 : 0);
}

// ---------------------------------------------------------------------------------------------
// K1: route + gate/up GEMV + SiLU*mul.  Items (distinct expert d, block of 16 rows of I).

template <int FMT, int MC>
__global__ __launch_bounds__(kDecThreads) void decode_up_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, int T, int E, int k, int H,
    int I, const uint8_t* __restrict__ gate_codes, const uint8_t* __restrict__ up_codes,
    const uint16_t* __restrict__ gate_scales, const uint16_t* __restrict__ up_scales,
    uint16_t* __restrict__ a16 /* [S][I] bf16 */, int* __restrict__ ids_ws,
    float* __restrict__ w_ws) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ RouteTable rt;
  const int tid = threadIdx.x, S = T * k;
  const int nb = H / 32, nblk = T * nb, nchunk = H / 64, rs = kChunkDwords * nchunk;
  uint32_t* pairs = reinterpret_cast<uint32_t*>(smem);
  float* cs = reinterpret_cast<float*>(smem + (size_t)T * rs * 4);
  // the first staging pass of x (two blocks per thread), loaded ahead of the routing
  u32x4_t xv[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int b = tid + p * kDecThreads;
    if (b < nblk) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)b * 32);
#pragma unroll
      for (int v = 0; v < 4; ++v) xv[p][v] = src[v];
    }
  }
  route_all_tokens(logits, T, E, k, rt.ids, rt.w);
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = tid; i < S; i += kDecThreads) { ids_ws[i] = rt.ids[i]; w_ws[i] = rt.w[i]; }
  build_table(rt, T, k, E, reinterpret_cast<int*>(smem));
  const int blocks = I / kUpRows;
  int it, end;
  item_range(rt.nd * blocks, it, end);
  if (it >= end) return;
  constexpr int CB = FMT == 2 ? 8 : 12;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15;
  const int rsub = wave * 4 + (lane >> 4);
  RowChunks<FMT, MC> gu[2];  // (gate row, up row); four waves per SIMD hide the load latency
  auto load_item = [&](int item) {
    const int d = item / blocks, n = (item % blocks) * kUpRows + rsub;
    const size_t row = (size_t)rt.dexp[d] * I + n;
    load_row_chunks<FMT, MC>(gu[0], gate_codes + row * nb * CB, gate_scales + row * nb, nchunk, c, 16);
    load_row_chunks<FMT, MC>(gu[1], up_codes + row * nb * CB, up_scales + row * nb, nchunk, c, 16);
  };
  load_item(it);
  // stage x (the routing table's scratch is dead now)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int b = tid + p * kDecThreads;
    if (b < nblk) stage_block<FMT>(xv[p], pairs + (b / nb) * rs, cs + (b / nb) * nb, b % nb);
  }
  for (int b = tid + 2 * kDecThreads; b < nblk; b += kDecThreads) {
    u32x4_t v[4];
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[i];
    stage_block<FMT>(v, pairs + (b / nb) * rs, cs + (b / nb) * nb, b % nb);
  }
  __syncthreads();
  for (; it < end; ++it) {
    const int d = it / blocks, n = (it % blocks) * kUpRows + rsub;
    const int Tp = rt.dtp[d];
    for (int tt = 0; tt < Tp; ++tt) {
      const int t = rt.dtok[d][tt];
      float acc[2];
      row_dots<FMT, MC, 2>(gu, nchunk, c, 16, pairs + t * rs, cs + t * nb, acc);
      const float gs = sum16(acc[0]), us = sum16(acc[1]);
      if (c == 0) {
        const float a = gs / (1.0f + expf(-gs)) * us;
        a16[(size_t)rt.dslot[d][tt] * I + n] = f32_to_bf16(a);
      }
    }
    if (it + 1 < end) load_item(it + 1);
  }
}

// ---------------------------------------------------------------------------------------------
// K2: down GEMV + combine.  Workgroup b owns rows [b R, (b+1) R) of H for every distinct expert;
// units (distinct expert d, row r), LPU lanes per unit.

template <int FMT, int MC, int LPU>
__global__ __launch_bounds__(kDnThreads) void decode_down_kernel(
    const uint16_t* __restrict__ a16, const int* __restrict__ ids_ws, const float* __restrict__ w_ws,
    int T, int E, int k, int H, int I, const uint8_t* __restrict__ down_codes,
    const uint16_t* __restrict__ down_scales, float* __restrict__ y, int accumulate) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ RouteTable rt;
  __shared__ float outs[kDecMaxS * kDecMaxR];  // [slot][r]
  const int tid = threadIdx.x, S = T * k;
  const int R = H / gridDim.x, h0 = blockIdx.x * R;
  const int nb = I / 32, nchunk = I / 64, rs = kChunkDwords * nchunk;
  uint32_t* pairs = reinterpret_cast<uint32_t*>(smem);
  float* cs = reinterpret_cast<float*>(smem + (size_t)S * rs * 4);
  if (tid < S) { rt.ids[tid] = ids_ws[tid]; rt.w[tid] = w_ws[tid]; }
  __syncthreads();
  build_table(rt, T, k, E, reinterpret_cast<int*>(smem));
  constexpr int CB = FMT == 2 ? 8 : 12;
  constexpr int kGroups = kDnThreads / LPU;
  const int U = rt.nd * R, g = tid / LPU, j = tid % LPU;
  RowChunks<FMT, MC> wr[2][1];
  auto load_unit = [&](int u, RowChunks<FMT, MC> (&rr)[1]) {
    const int d = u / R, r = u % R;
    const size_t row = (size_t)rt.dexp[d] * H + h0 + r;
    load_row_chunks<FMT, MC>(rr[0], down_codes + row * nb * CB, down_scales + row * nb, nchunk, j, LPU);
  };
  if (g < U) load_unit(g, wr[0]);
  if (g + kGroups < U) load_unit(g + kGroups, wr[1]);
  // stage every slot's intermediate a (the routing table's scratch is dead now)
  for (int b = tid; b < S * nb; b += kDnThreads) {
    const int s = b / nb, blk = b % nb;
    u32x4_t v[4];
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a16 + (size_t)s * I + blk * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[i];
    stage_block<FMT>(v, pairs + s * rs, cs + s * nb, blk);
  }
  __syncthreads();
  auto compute_unit = [&](int u, const RowChunks<FMT, MC> (&rr)[1]) {
    const int d = u / R, r = u % R;
    const int Tp = rt.dtp[d];  // uniform over the unit's lanes
    for (int tt = 0; tt < Tp; ++tt) {
      const int slot = rt.dslot[d][tt];
      float acc[1];
      row_dots<FMT, MC, 1>(rr, nchunk, j, LPU, pairs + slot * rs, cs + slot * nb, acc);
      const float v = LPU == 4 ? sum4(acc[0]) : sum16(acc[0]);
      if (j == 0) outs[slot * R + r] = v;
    }
  };
  for (int u = g; u < U; u += 2 * kGroups) {
    compute_unit(u, wr[0]);
    if (u + 2 * kGroups < U) load_unit(u + 2 * kGroups, wr[0]);
    if (u + kGroups < U) {
      compute_unit(u + kGroups, wr[1]);
      if (u + 3 * kGroups < U) load_unit(u + 3 * kGroups, wr[1]);
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
  const size_t st = (size_t)T * staged_row_bytes(H), sc = (size_t)2 * E * 4;
  return st > sc ? st : sc;
}
static size_t dn_lds_bytes(int T, int E, int k, int I) {
  const size_t st = (size_t)T * k * staged_row_bytes(I), sc = (size_t)2 * E * 4;
  return st > sc ? st : sc;
}
constexpr size_t kDecLdsLimit = 160 * 1024 - 16 * 1024;  // dynamic LDS beside the static tables

bool decode_fits(int T, int E, int k, int H, int I) {
  if (T < 1 || T > kDecMaxT || T * k > kDecMaxS || E > 1024) return false;
  if (H % 256 || H > 4096 || I % 128 || I > 4096) return false;
  return up_lds_bytes(T, E, H) <= kDecLdsLimit && dn_lds_bytes(T, E, k, I) <= kDecLdsLimit;
}

// Workspace: ids [S] int32 | w [S] fp32 | a [S][I] bf16
size_t decode_workspace_bytes(int T, int E, int k, int H, int I) {
  (void)E; (void)H;
  const size_t S = (size_t)T * k;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return up(S * 4) + up(S * 4) + up(S * I * 2);
}

template <typename K>
static void allow_lds(K kernel) {
  hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecLdsLimit);
}

template <int F>
static void allow_all_decode_lds() {
  allow_lds(decode_up_kernel<F, 1>); allow_lds(decode_up_kernel<F, 2>);
  allow_lds(decode_up_kernel<F, 3>); allow_lds(decode_up_kernel<F, 4>);
  allow_lds(decode_down_kernel<F, 1, 4>); allow_lds(decode_down_kernel<F, 2, 4>);
  allow_lds(decode_down_kernel<F, 3, 4>); allow_lds(decode_down_kernel<F, 4, 4>);
  allow_lds(decode_down_kernel<F, 2, 16>); allow_lds(decode_down_kernel<F, 3, 16>);
  allow_lds(decode_down_kernel<F, 4, 16>);
}

hipError_t launch_decode(int fmt, const uint16_t* x, const float* logits, int T, int E, int k,
                         int H, int I, const void* gate_codes, const void* up_codes,
                         const void* down_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, const uint16_t* down_scales, float* y,
                         int accumulate, int* ids_out, float* w_out, void* ws, hipStream_t s) {
  if (!decode_fits(T, E, k, H, I)) return hipErrorInvalidValue;
  static std::once_flag once;
  std::call_once(once, [] { allow_all_decode_lds<2>(); allow_all_decode_lds<3>(); });
  const size_t S = (size_t)T * k;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  int* ids = ids_out ? ids_out : reinterpret_cast<int*>(p);
  p += up(S * 4);
  float* w = w_out ? w_out : reinterpret_cast<float*>(p);
  p += up(S * 4);
  uint16_t* a16 = reinterpret_cast<uint16_t*>(p);
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  const size_t lds_up = up_lds_bytes(T, E, H), lds_dn = dn_lds_bytes(T, E, k, I);
  const int grid_up = 1024;  // four 4-wave workgroups per CU
  const int mc_up = (H / 64 + 15) / 16;                 // 1..4 chunks per lane (16 lanes per row)
  const int nch_dn = I / 64;
  const int lpu = nch_dn <= 16 ? 4 : 16;                 // lanes per down row
  const int mc_dn = (nch_dn + lpu - 1) / lpu;            // 1..4
#define STRATA_UP(F, M)                                                                          \
  decode_up_kernel<F, M><<<grid_up, kDecThreads, lds_up, s>>>(x, logits, T, E, k, H, I, gc, uc,   \
                                                              gate_scales, up_scales, a16, ids, w)
#define STRATA_DN(F, M, L)                                                                       \
  decode_down_kernel<F, M, L><<<kDnGrid, kDnThreads, lds_dn, s>>>(a16, ids, w, T, E, k, H, I, dc, \
                                                                   down_scales, y, accumulate)
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

}  // namespace strata
