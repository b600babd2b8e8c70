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

// Wave-wide float sum, result uniform: row sums by DPP, then the rows folded into lane 63 by the
// two row broadcasts (no LDS round trip, unlike a shuffle butterfly).
STRATA_DEVICE float wave_sum_dpp(float v) {
  v = sum16(v);
  v += __builtin_bit_cast(float, dpp_u<0x142, 0xA>(__builtin_bit_cast(uint32_t, v), 0u));  // row_bcast:15
  v += __builtin_bit_cast(float, dpp_u<0x143, 0xC>(__builtin_bit_cast(uint32_t, v), 0u));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Inclusive prefix sum of ints across the wave's lanes: shifts within each row of 16 lanes, then
// the row broadcasts carry each row's total into the rows above it.
STRATA_DEVICE int wave_scan_dpp(int v) {
  v += (int)dpp_u<0x111>((uint32_t)v, 0u);  // row_shr:1
  v += (int)dpp_u<0x112>((uint32_t)v, 0u);  // row_shr:2
  v += (int)dpp_u<0x114>((uint32_t)v, 0u);  // row_shr:4
  v += (int)dpp_u<0x118>((uint32_t)v, 0u);  // row_shr:8
  v += (int)dpp_u<0x142, 0xA>((uint32_t)v, 0u);  // row_bcast:15 into rows 1 and 3
  v += (int)dpp_u<0x143, 0xC>((uint32_t)v, 0u);  // row_bcast:31 into rows 2 and 3
  return v;
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

// Orders this wave's LDS accesses across its lanes.  The LDS executes one wave's instructions in
// issue order, so keeping the compiler from moving accesses across this point suffices (wavefront
// scope: no wait is emitted).
STRATA_DEVICE void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Top-k selection over the wave's per-lane sorted entries (composite keys, all distinct among real
// entries, 0 = empty).  On lane j < k it leaves the j-th largest key's logit key and expert.
//
// Threshold and rank: the k-th largest of the 64 lane heads, tau, is at most the k-th largest
// entry overall (k heads are >= tau), so the top k are among the entries >= tau: usually k to
// k + 5 of them, at most k * NPL.  They are gathered in LDS and each one's rank among them is
// counted; ranks 0..k-1 are the selection.  Returns false (LDS untouched beyond this wave's 80
// entries, c unchanged) when more than 64 entries pass, left to select_rounds.  Real heads number
// min(E, 64) >= k and are distinct, so exactly one lane's head has k - 1 heads above it.
template <int NPL>
STRATA_DEVICE bool select_threshold(const uint64_t (&c)[NPL], int k, uint64_t* lds,
                                    uint32_t& my_key, int& my_i) {
  typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const uint64_t h = c[0];
  lds[lane] = h;
  wave_lds_sync();
  int above = 0;
#pragma unroll 8
  for (int j = 0; j < 64; j += 2) {
    const u64x2_t p = *reinterpret_cast<const u64x2_t*>(lds + j);
    above += (p[0] > h) + (p[1] > h);
  }
  const int tl = __ffsll((unsigned long long)__ballot(above == k - 1)) - 1;
  const uint64_t tau = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(h >> 32), tl) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)h, tl);
  wave_lds_sync();
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {  // lanes are sorted: entry i passes only where entry i - 1 did
    const bool in = c[i] >= tau;
    const uint64_t b = __ballot(in);
    if (b == 0) break;
    const int cnt = __popcll(b);
    if (n + cnt > 64) return false;
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
    if (in) lds[n + below] = c[i];
    n += cnt;
  }
  wave_lds_sync();
  const uint64_t mine = lds[lane < n ? lane : 0];
  int r = 0;
  for (int j = 0; j < n; ++j) r += lds[j] > mine;
  wave_lds_sync();
  if (lane < n && r < k) lds[64 + r] = mine;
  wave_lds_sync();
  const uint64_t sel = lds[64 + (lane < k ? lane : 0)];
  my_key = lane < k ? (uint32_t)(sel >> 32) : 0u;
  my_i = lane < k ? (int)~(uint32_t)sel : 0;
  return true;
}

// The same selection by k rounds of a wave-wide arg-max over the lanes' heads, the winning lane
// popping its head (c is consumed).
template <int NPL>
STRATA_DEVICE void select_rounds(uint64_t (&c)[NPL], int k, uint32_t& my_key, int& my_i) {
  const int lane = threadIdx.x & 63;
  my_key = 0;
  my_i = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hk = (uint32_t)(c[0] >> 32);
    const uint32_t m = wave_max_u32(hk);
    const bool cand = hk == m;
    const uint64_t ball = __ballot(cand);
    int win;
    if (__popcll(ball) == 1) {  // the usual case: one lane holds the maximum
      const int wl = __ffsll((unsigned long long)ball) - 1;
      win = (int)~(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c[0], wl);
    } else {                    // equal logits in several lanes: lowest expert index
      win = (int)~wave_max_u32(cand ? (uint32_t)c[0] : 0u);
    }
    if (lane == j) { my_key = m; my_i = win; }
    const bool pop = lane == (win & 63);
#pragma unroll
    for (int i = 0; i + 1 < NPL; ++i) c[i] = pop ? c[i + 1] : c[i];
    c[NPL - 1] = pop ? 0ull : c[NPL - 1];
  }
}

// Top-k of one token by one wave: the k largest logits, equal logits to the lower expert index;
// weights = softmax over the k kept logits (the router kernel's rule).  Each lane sorts its own
// entries once, then select_threshold (select_rounds where it declines).  lds: 80 uint64 of LDS
// (16-byte aligned) used by this wave alone.
template <int NPL>
STRATA_DEVICE void select_token_wave(TokenKeys<NPL>& tk, int E, int k, int* ids_out,
                                     float* w_out, uint64_t* lds) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    tk.c[i] = e < E ? ((uint64_t)route_key(tk.v[i]) << 32) | (uint32_t)~e : 0ull;
  }
  sort_lane_desc<NPL>(tk.c);
  uint32_t my_key;
  int my_i;
  if (!select_threshold<NPL>(tk.c, k, lds, my_key, my_i)) select_rounds<NPL>(tk.c, k, my_key, my_i);
  const float top = key_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
  const float ex = lane < k ? expf(key_value(my_key) - top) : 0.0f;
  const float den = wave_sum_dpp(ex);
  if (lane < k) {
    ids_out[lane] = my_i;
    w_out[lane] = ex / den;
  }
}

}  // namespace strata
