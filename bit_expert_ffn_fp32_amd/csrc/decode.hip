// Decode / verify path for T <= 8 tokens: bandwidth-bound GEMVs over the touched experts.
//
// The pages verify up to 3 drafted tokens plus one in a single pass over the layers ("Strata - the
// details", How it works / speculation) and note that decode is bound by memory bandwidth
// ("Two-Day Port, 8x Faster Prefill: Strata Engine Benchmarked", Why Prefill Matters).  Every
// touched expert's packed weights are streamed from HBM exactly once and applied to every token
// that picked it, so HBM bytes equal the packed size of the touched experts.
//
// Kernels: route (shared with the prefill path) -> up (gate/up GEMV + SiLU*mul) -> down (GEMV per
// slot, fp32) -> combine (weighted sum in slot order).  The up and down grids are (row block,
// slot); a slot whose expert already appeared at a lower slot index exits at once, and the first
// slot of each expert serves all tokens that picked it.
//
// Arithmetic.  Weights are exact: a 2-bit code q enters a bf16 dot product as 2 + q/2 (exact,
// built with one shift and one and-or from the packed word), a 3-bit code as 4 + q/2 for
// q in 0..7 (also exact), and the fp16 block scale is applied in fp32:
//   sum_i (q_i - 1.5) x_i = 2 * sum_i (2 + q_i/2) x_i - 5.5 * sum_i x_i      (2-bit)
//   sum_i (q_i - 3.5) x_i = 2 * sum_i (4 + q_i/2) x_i - 11.5 * sum_i x_i     (3-bit)
// with the x sums taken once per 16-value word.  x stays bf16 (the input precision); the SiLU*mul
// intermediate is rounded to bf16 for the down GEMV; outputs stay fp32.
//
// Pairing: a 32-bit word of 2-bit codes holds 16 codes; bf16 pair m (m = 0..7) holds codes m and
// m+8 (bits 2m and 2m+16 of the word), so each pair is one shift + and-or.  The activations are
// staged in LDS in the same pairing (P16 = {0,8,1,9,...,7,15} within each group of 16).
#include "common.hpp"
#include "kernels.hpp"

namespace strata {

constexpr int kDecThreads = 256;       // 4 waves
constexpr int kDecRowsPerWave = 4;     // 16 lanes per row
constexpr int kDecRows = 16;           // rows per workgroup
constexpr int kDecMaxT = 8;

// Codes of one 16-value word -> 8 bf16 pairs of (offset + q/2), pair m = codes (m, m+8).
// 2-bit: bf16(2 + q/2) = 0x4000 | q << 5.
STRATA_DEVICE void q2_word_pairs(uint32_t w, uint32_t out[8]) {
  out[0] = ((w << 5) & 0x00600060u) | 0x40004000u;
  out[1] = ((w << 3) & 0x00600060u) | 0x40004000u;
  out[2] = ((w << 1) & 0x00600060u) | 0x40004000u;
  out[3] = ((w >> 1) & 0x00600060u) | 0x40004000u;
  out[4] = ((w >> 3) & 0x00600060u) | 0x40004000u;
  out[5] = ((w >> 5) & 0x00600060u) | 0x40004000u;
  out[6] = ((w >> 7) & 0x00600060u) | 0x40004000u;
  out[7] = ((w >> 9) & 0x00600060u) | 0x40004000u;
}

// 3-bit: 16 codes = 48 bits (lo 32 + hi 16 bits); bf16(4 + q/2) = 0x4080 | q << 4.
// Pair m = codes (m, m+8).
STRATA_DEVICE void q3_word_pairs(uint32_t lo, uint32_t hi, uint32_t out[8]) {
  const uint64_t v = (uint64_t)lo | ((uint64_t)hi << 32);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t qa = (uint32_t)(v >> (3 * m)) & 7u;
    const uint32_t qb = (uint32_t)(v >> (3 * (m + 8))) & 7u;
    out[m] = (0x4080u | (qa << 4)) | ((0x4080u | (qb << 4)) << 16);
  }
}

// Reads word wi (16 values) of a packed row: 2-bit words are 4 bytes; 3-bit words are 6 bytes
// (bits 48*(wi%2) .. of the block's 96 bits).
template <int FMT>
STRATA_DEVICE void load_word(const uint8_t* row, int wi, uint32_t& lo, uint32_t& hi) {
  if constexpr (FMT == 2) {
    lo = reinterpret_cast<const uint32_t*>(row)[wi];
    hi = 0;
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row + (size_t)(wi >> 1) * 12 + (wi & 1) * 6);
    lo = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
    hi = p[2];
  }
}

template <int FMT>
STRATA_DEVICE float word_dot(uint32_t lo, uint32_t hi, const uint32_t* xp) {
  uint32_t pr[8];
  if constexpr (FMT == 2) q2_word_pairs(lo, pr);
  else q3_word_pairs(lo, hi, pr);
  float p = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr[m]),
                                        __builtin_bit_cast(bf16x2_t, xp[m]), p, false);
  return p;
}

// LDS staging of T' activation rows in P16 pairing, plus per-word sums.
// src rows are bf16 [K]; dst pairs [T'][K/2] dwords; sums [T'][K/16].
STRATA_DEVICE void stage_pairs(const uint16_t* const* src, int Tp, int K, uint32_t* pairs,
                               float* sums) {
  const int words = K / 16;
  for (int idx = threadIdx.x; idx < Tp * words; idx += kDecThreads) {
    const int tt = idx / words, wi = idx % words;
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(src[tt] + (size_t)wi * 16);
    const u32x4_t a = p[0], b = p[1];
    const uint32_t e[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};  // values 2i, 2i+1
    float s = 0.0f;
    uint32_t* dst = pairs + ((size_t)tt * words + wi) * 8;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      // value m (element m of the 16) and value m+8
      const uint32_t vm = (m & 1) ? (e[m >> 1] >> 16) : (e[m >> 1] & 0xFFFFu);
      const uint32_t vn = (m & 1) ? (e[4 + (m >> 1)] >> 16) : (e[4 + (m >> 1)] & 0xFFFFu);
      dst[m] = vm | (vn << 16);
      s += bf16_to_f32((uint16_t)vm) + bf16_to_f32((uint16_t)vn);
    }
    sums[(size_t)tt * words + wi] = s;
  }
}

// Finds this workgroup's expert (first slot of it) and the tokens that picked it.  Called by
// every thread; ids_l is LDS of at least T*k ints.  Returns T' (0 if the slot is not the first
// one of its expert).
STRATA_DEVICE int decode_claim(const int* ids, int T, int k, int* ids_l, int* tok, int* slot,
                               int* info) {
  const int S = T * k;
  for (int i = threadIdx.x; i < S; i += blockDim.x) ids_l[i] = ids[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    const int s = blockIdx.y;
    const int e = ids_l[s];
    bool first = true;
    for (int s2 = 0; s2 < s; ++s2) first = first && ids_l[s2] != e;
    int Tp = 0;
    if (first)
      for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
          if (ids_l[t * k + j] == e) { tok[Tp] = t; slot[Tp] = t * k + j; ++Tp; }
    info[0] = Tp;
    info[1] = e;
  }
  __syncthreads();
  return info[0];
}

STRATA_DEVICE int p16pos(int n) { return (n & ~15) | ((n & 7) << 1) | ((n >> 3) & 1); }

// ---------------------------------------------------------------------------------------------

template <int FMT>
__global__ __launch_bounds__(kDecThreads) void decode_up_kernel(
    const uint16_t* __restrict__ x, const int* __restrict__ ids, int T, int k, int H, int I,
    const uint8_t* __restrict__ gate_codes, const uint8_t* __restrict__ up_codes,
    const uint16_t* __restrict__ gate_scales, const uint16_t* __restrict__ up_scales,
    uint32_t* __restrict__ a_pairs /* [S][I/2] bf16 pairs in P16 order */) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int tok[kDecMaxT], slot[kDecMaxT], info[2], ids_l[kDecMaxT * 16];
  const int Tp = decode_claim(ids, T, k, ids_l, tok, slot, info);
  const int e = info[1];
  if (Tp == 0) return;
  const int words = H / 16;
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem);
  float* sx = reinterpret_cast<float*>(smem + (size_t)Tp * words * 32);
  {
    const uint16_t* src[kDecMaxT];
    for (int tt = 0; tt < Tp; ++tt) src[tt] = x + (size_t)tok[tt] * H;
    stage_pairs(src, Tp, H, xp, sx);
  }
  __syncthreads();
  constexpr int CB = FMT == 2 ? 8 : 12;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int n = blockIdx.x * kDecRows + wave * kDecRowsPerWave + (lane >> 4);
  const int nbh = H / 32;
  const size_t row = (size_t)e * I + n;
  const uint8_t* gr = gate_codes + row * nbh * CB;
  const uint8_t* ur = up_codes + row * nbh * CB;
  const uint16_t* gsr = gate_scales + row * nbh;
  const uint16_t* usr = up_scales + row * nbh;
  const float c0x2 = FMT == 2 ? 5.5f : 11.5f;
  float g[kDecMaxT], u[kDecMaxT];
#pragma unroll
  for (int tt = 0; tt < kDecMaxT; ++tt) { g[tt] = 0.0f; u[tt] = 0.0f; }
  for (int wi = c; wi < words; wi += 16) {
    uint32_t glo, ghi, ulo, uhi;
    load_word<FMT>(gr, wi, glo, ghi);
    load_word<FMT>(ur, wi, ulo, uhi);
    const float dg = f16_to_f32(gsr[wi >> 1]), du = f16_to_f32(usr[wi >> 1]);
#pragma unroll
    for (int tt = 0; tt < kDecMaxT; ++tt) {
      if (tt < Tp) {
        const uint32_t* xw = xp + ((size_t)tt * words + wi) * 8;
        const float s = sx[(size_t)tt * words + wi];
        const float pg = word_dot<FMT>(glo, ghi, xw);
        const float pu = word_dot<FMT>(ulo, uhi, xw);
        g[tt] = __builtin_fmaf(dg, __builtin_fmaf(2.0f, pg, -c0x2 * s), g[tt]);
        u[tt] = __builtin_fmaf(du, __builtin_fmaf(2.0f, pu, -c0x2 * s), u[tt]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < kDecMaxT; ++tt) {
    if (tt < Tp) {
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        g[tt] += __shfl_xor(g[tt], off);
        u[tt] += __shfl_xor(u[tt], off);
      }
    }
  }
  if (c == 0) {
    uint16_t* ap = reinterpret_cast<uint16_t*>(a_pairs);
    const int pos = p16pos(n);
    for (int tt = 0; tt < Tp; ++tt) {
      const float a = g[tt] / (1.0f + expf(-g[tt])) * u[tt];
      ap[(size_t)slot[tt] * I + pos] = f32_to_bf16(a);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kDecThreads) void decode_down_kernel(
    const uint32_t* __restrict__ a_pairs, const int* __restrict__ ids, int T, int k, int H, int I,
    const uint8_t* __restrict__ down_codes, const uint16_t* __restrict__ down_scales,
    float* __restrict__ out32 /* [S][H] */) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int tok[kDecMaxT], slot[kDecMaxT], info[2], ids_l[kDecMaxT * 16];
  const int Tp = decode_claim(ids, T, k, ids_l, tok, slot, info);
  const int e = info[1];
  if (Tp == 0) return;
  const int words = I / 16;
  uint32_t* ap = reinterpret_cast<uint32_t*>(smem);
  float* sa = reinterpret_cast<float*>(smem + (size_t)Tp * words * 32);
  // a is already in P16 pairing: copy and form the word sums
  for (int idx = threadIdx.x; idx < Tp * words; idx += kDecThreads) {
    const int tt = idx / words, wi = idx % words;
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(a_pairs + ((size_t)slot[tt] * I) / 2 + wi * 8);
    const u32x4_t a = p[0], b = p[1];
    uint32_t* dst = ap + ((size_t)tt * words + wi) * 8;
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      dst[m] = a[m];
      dst[m + 4] = b[m];
      s += bf16_to_f32((uint16_t)(a[m] & 0xFFFFu)) + bf16_to_f32((uint16_t)(a[m] >> 16));
      s += bf16_to_f32((uint16_t)(b[m] & 0xFFFFu)) + bf16_to_f32((uint16_t)(b[m] >> 16));
    }
    sa[(size_t)tt * words + wi] = s;
  }
  __syncthreads();
  constexpr int CB = FMT == 2 ? 8 : 12;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int h = blockIdx.x * kDecRows + wave * kDecRowsPerWave + (lane >> 4);
  const int nbi = I / 32;
  const size_t row = (size_t)e * H + h;
  const uint8_t* dr = down_codes + row * nbi * CB;
  const uint16_t* dsr = down_scales + row * nbi;
  const float c0x2 = FMT == 2 ? 5.5f : 11.5f;
  float o[kDecMaxT];
#pragma unroll
  for (int tt = 0; tt < kDecMaxT; ++tt) o[tt] = 0.0f;
  for (int wi = c; wi < words; wi += 16) {
    uint32_t lo, hi;
    load_word<FMT>(dr, wi, lo, hi);
    const float d = f16_to_f32(dsr[wi >> 1]);
#pragma unroll
    for (int tt = 0; tt < kDecMaxT; ++tt) {
      if (tt < Tp) {
        const float p = word_dot<FMT>(lo, hi, ap + ((size_t)tt * words + wi) * 8);
        o[tt] = __builtin_fmaf(d, __builtin_fmaf(2.0f, p, -c0x2 * sa[(size_t)tt * words + wi]), o[tt]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < kDecMaxT; ++tt) {
    if (tt < Tp) {
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) o[tt] += __shfl_xor(o[tt], off);
    }
  }
  if (c == 0)
    for (int tt = 0; tt < Tp; ++tt) out32[(size_t)slot[tt] * H + h] = o[tt];
}

__global__ void decode_combine_kernel(const float* __restrict__ out32, const float* __restrict__ w,
                                      int T, int k, int H, float* __restrict__ y, int accumulate) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * H) return;
  const int t = i / H, h = i % H;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s = __builtin_fmaf(w[t * k + j], out32[((size_t)t * k + j) * H + h], s);
  y[i] = accumulate ? y[i] + s : s;
}

// Workspace: ids [T*k] int32 | w [T*k] fp32 | a pairs [T*k][I] bf16 | out32 [T*k][H] fp32
size_t decode_workspace_bytes(int T, int E, int k, int H, int I) {
  (void)E;
  const size_t S = (size_t)T * k;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return up(S * 4) + up(S * 4) + up(S * I * 2) + up(S * H * 4);
}

hipError_t launch_decode(int fmt, const uint16_t* x, const float* logits, int T, int E, int k,
                         int H, int I, const void* gate_codes, const void* up_codes,
                         const void* down_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, const uint16_t* down_scales, float* y,
                         int accumulate, int* ids_out, float* w_out, void* ws, hipStream_t s) {
  const size_t S = (size_t)T * k;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  int* ids = ids_out ? ids_out : reinterpret_cast<int*>(p);
  p += up(S * 4);
  float* w = w_out ? w_out : reinterpret_cast<float*>(p);
  p += up(S * 4);
  uint32_t* a_pairs = reinterpret_cast<uint32_t*>(p);
  p += up(S * I * 2);
  float* out32 = reinterpret_cast<float*>(p);
  hipError_t err = launch_route(logits, T, E, k, ids, w, s);
  if (err != hipSuccess) return err;
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  const size_t lds_up = (size_t)T * (H / 16) * (32 + 4);
  const size_t lds_dn = (size_t)T * (I / 16) * (32 + 4);
  dim3 gu(I / kDecRows, (unsigned)S), gd(H / kDecRows, (unsigned)S);
  if (fmt == 2) {
    decode_up_kernel<2><<<gu, kDecThreads, lds_up, s>>>(x, ids, T, k, H, I, gc, uc, gate_scales,
                                                        up_scales, a_pairs);
    decode_down_kernel<2><<<gd, kDecThreads, lds_dn, s>>>(a_pairs, ids, T, k, H, I, dc, down_scales,
                                                          out32);
  } else {
    decode_up_kernel<3><<<gu, kDecThreads, lds_up, s>>>(x, ids, T, k, H, I, gc, uc, gate_scales,
                                                        up_scales, a_pairs);
    decode_down_kernel<3><<<gd, kDecThreads, lds_dn, s>>>(a_pairs, ids, T, k, H, I, dc, down_scales,
                                                          out32);
  }
  decode_combine_kernel<<<(T * H + 255) / 256, 256, 0, s>>>(out32, w, T, k, H, y, accumulate);
  return hipGetLastError();
}

}  // namespace strata
