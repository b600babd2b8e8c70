// Wave-level helpers shared by the routing kernels: DPP reductions and the one-wave top-k
// selection of a token's experts.
#pragma once

#include "common.hpp"

namespace strata {

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

// Wave-wide max of unsigned keys / min of ints, result uniform (read from lane 63).  The DPP
// moves take the identity of the operation as their fill value so that each step folds into one
// DPP-modified max / min.
template <int CTRL, int ROW_MASK = 0xF>
STRATA_DEVICE uint32_t dpp_u(uint32_t v, uint32_t fill) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROW_MASK, 0xF, false);
}
STRATA_DEVICE uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v, 0u));
  v = max(v, dpp_u<0x4E>(v, 0u));
  v = max(v, dpp_u<0x124>(v, 0u));
  v = max(v, dpp_u<0x128>(v, 0u));
  v = max(v, dpp_u<0x142, 0xA>(v, 0u));  // row_bcast:15
  v = max(v, dpp_u<0x143, 0xC>(v, 0u));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
STRATA_DEVICE int wave_min_i(int v) {
  v = min(v, (int)dpp_u<0xB1>((uint32_t)v, 0x7FFFFFFFu));
  v = min(v, (int)dpp_u<0x4E>((uint32_t)v, 0x7FFFFFFFu));
  v = min(v, (int)dpp_u<0x124>((uint32_t)v, 0x7FFFFFFFu));
  v = min(v, (int)dpp_u<0x128>((uint32_t)v, 0x7FFFFFFFu));
  v = min(v, (int)dpp_u<0x142, 0xA>((uint32_t)v, 0x7FFFFFFFu));
  v = min(v, (int)dpp_u<0x143, 0xC>((uint32_t)v, 0x7FFFFFFFu));
  return __builtin_amdgcn_readlane(v, 63);
}

// Order-preserving map of a logit to an unsigned key (-0 is first made +0, so equal logits get
// equal keys; every finite logit maps to a key above 0, which marks an empty entry), and back.
STRATA_DEVICE uint32_t route_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
STRATA_DEVICE float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// One token's logits, lane l holding experts l, l + 64, ...  The loads are unconditional
// (clamped addresses) so that they are all in flight together.
template <int NPL>
struct TokenKeys {
  float v[NPL];       // raw logits, converted once they have arrived
  uint64_t c[NPL];    // (key << 32) | ~expert: larger is preferred, ties to the lower expert
};
template <int NPL>
STRATA_DEVICE void load_token_logits(const float* __restrict__ row, int E, TokenKeys<NPL>& tk) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NPL; ++i) tk.v[i] = row[min(lane + 64 * i, E - 1)];
}

// Sorts the lane's entries, largest first (Batcher's odd-even merge network; NPL a power of 2).
template <int NPL>
STRATA_DEVICE void sort_lane_desc(uint64_t (&c)[NPL]) {
#pragma unroll
  for (int p = 1; p < NPL; p <<= 1)
#pragma unroll
    for (int kk = p; kk >= 1; kk >>= 1)
#pragma unroll
      for (int j = kk % p; j + kk < NPL; j += 2 * kk)
#pragma unroll
        for (int i = 0; i < kk && i + j + kk < NPL; ++i)
          if ((i + j) / (2 * p) == (i + j + kk) / (2 * p)) {
            const uint64_t a = c[i + j], b = c[i + j + kk];
            const bool sw = b > a;
            c[i + j] = sw ? b : a;
            c[i + j + kk] = sw ? a : b;
          }
}

// Top-k of one token by one wave: k rounds of "largest remaining logit, equal logits to the lower
// expert index"; weights = softmax over the k kept logits (the router kernel's rule).  Each lane
// sorts its own entries once; a round takes the maximum of the lanes' heads and the winning lane
// pops its head.
template <int NPL>
STRATA_DEVICE void select_token_wave(TokenKeys<NPL>& tk, int E, int k, int* ids_out,
                                     float* w_out) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    tk.c[i] = e < E ? ((uint64_t)route_key(tk.v[i]) << 32) | (uint32_t)~e : 0ull;
  }
  sort_lane_desc<NPL>(tk.c);
  uint32_t my_key = 0;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hk = (uint32_t)(tk.c[0] >> 32);
    const uint32_t m = wave_max_u32(hk);
    const bool cand = hk == m;
    const uint64_t ball = __ballot(cand);
    int win;
    if (__popcll(ball) == 1) {  // the usual case: one lane holds the maximum
      const int wl = __ffsll((unsigned long long)ball) - 1;
      win = (int)~(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)tk.c[0], wl);
    } else {                    // equal logits in several lanes: lowest expert index
      win = (int)~wave_max_u32(cand ? (uint32_t)tk.c[0] : 0u);
    }
    if (lane == j) { my_key = m; my_i = win; }
    const bool pop = lane == (win & 63);
#pragma unroll
    for (int i = 0; i + 1 < NPL; ++i) tk.c[i] = pop ? tk.c[i + 1] : tk.c[i];
    tk.c[NPL - 1] = pop ? 0ull : tk.c[NPL - 1];
  }
  const float top = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
  const float ex = lane < k ? expf(key_value(my_key) - top) : 0.0f;
  const float den = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_i;
    w_out[lane] = ex / den;
  }
}

}  // namespace strata
