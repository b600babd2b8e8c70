// Prefill path: grouped expert GEMMs on the matrix cores, combine, RMSNorm.
//
// The pages name the expert matrix multiply as the heaviest computation of the model and say the
// low-bit blocks are dequantized on the fly inside it ("Two-Day Port, 8x Faster Prefill: Strata
// Engine Benchmarked", Where Strata Is Fast); a larger prefill batch lets every expert's weights
// serve more tokens (same section).  Here every work unit is weight-stationary: one (expert,
// output slice) pair streams its packed 2- or 3-bit blocks once per chunk of up to 256 of the
// expert's tokens, decodes them in registers and feeds v_mfma_f32_32x32x16_f16 with fp32
// accumulation.
//
// Numerics.  A weight is d * (q - c0) with an fp16 scale d.  The decoder forms the fp16 product
// fp16(d * (q - c0)) with one round-to-nearest-even (exact whenever q - c0 = +-0.5; otherwise the
// product needs 12-13 significant bits and is rounded to fp16's 11).  Activations enter the
// matrix cores as fp16 (bf16 inputs convert exactly within fp16's normal range); the SiLU*mul
// intermediate is stored as fp16 and expert outputs as bf16.
//
// Operand order.  Within every group of 8 consecutive reduction indices the GEMM feeds the
// matrix cores the order P8 = {0,4,1,5,2,6,3,7}: the decoder then produces each fp16 pair from one
// byte-table lookup (v_perm_b32).  The activations are stored in the same order (x by the
// conversion kernel, the intermediate by the up-projection epilogue), so the sums are unchanged.
//
// Work distribution.  Units (chunk, slice) are numbered so that the units of one expert are
// consecutive; blockIdx is mapped so that consecutive units run on the same XCD (workgroups are
// dealt to the 8 XCDs round-robin), which keeps an expert's weights and its tokens' activations
// in that XCD's L2 while all of its slices run.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace strata {

constexpr int kGemmThreads = 256;               // 4 waves, one per SIMD
constexpr int kKC = 128;                        // reduction indices per pipeline stage
constexpr int kLdsRow = kKC + 8;                // halfs per LDS row (16-byte pad: no bank conflicts)
constexpr int kFrags = kChunkRows / 32;         // 32-row fragments per chunk
constexpr int kLdsTile = kChunkRows * kLdsRow;  // halfs per stage buffer
constexpr size_t kGemmLds = 2 * kLdsTile * sizeof(uint16_t) + kChunkRows * sizeof(int);

STRATA_DEVICE int p8inv(int m) { return ((m & 3) << 1) | (m >> 2); }  // position of index m

// ---------------------------------------------------------------------------------------------
// Block decoders.  A lane owns two consecutive blocks (64 reduction indices) of one weight row per
// stage and produces, for stage step s (0..7), the 8 fp16 weights of indices 8s .. 8s+7 of that
// 64-range in P8 order.

struct Q2Tab {
  uint32_t lo, hi;  // byte q of lo/hi = low/high byte of fp16(d * (q - 1.5))
};

STRATA_DEVICE Q2Tab q2_table(uint16_t dbits) {
  const _Float16 d = __builtin_bit_cast(_Float16, dbits);
  const float df = (float)d;
  const uint32_t w0 = __builtin_bit_cast(uint16_t, (_Float16)(df * -1.5f));
  const uint32_t w1 = __builtin_bit_cast(uint16_t, (_Float16)(df * -0.5f));
  const uint32_t w2 = __builtin_bit_cast(uint16_t, (_Float16)(df * 0.5f));
  const uint32_t w3 = __builtin_bit_cast(uint16_t, (_Float16)(df * 1.5f));
  const uint32_t p01 = w0 | (w1 << 16), p23 = w2 | (w3 << 16);
  return Q2Tab{__builtin_amdgcn_perm(p23, p01, 0x06040200u), __builtin_amdgcn_perm(p23, p01, 0x07050301u)};
}

// codes: the lane's 16 code bytes (2 blocks); bytes 2s, 2s+1 hold the 8 codes of step s.
STRATA_DEVICE half8_t q2_decode(const u32x4_t& codes, int s, const Q2Tab& tab) {
  const uint32_t word = codes[s >> 1];
  const uint32_t X = __builtin_amdgcn_perm(word, word, (s & 1) ? 0x03030202u : 0x01010000u);
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sel = ((X >> (2 * i)) & 0x03030303u) | 0x04000400u;
    r[i] = __builtin_amdgcn_perm(tab.hi, tab.lo, sel);
  }
  return __builtin_bit_cast(half8_t, r);
}

// 3-bit codes: the lane's 24 code bytes (2 blocks of 12) as 6 words; step s covers codes
// 8(s%4) .. 8(s%4)+7 of block s/4, i.e. 24 bits at bit offset 24(s%4) of that block.
STRATA_DEVICE half8_t q3_decode(const uint32_t* cw, int s, float d) {
  const int base = (s >> 2) * 3;
  const int o = 24 * (s & 3);
  const uint32_t lo = cw[base + (o >> 5)];
  const uint32_t hi = cw[base + ((o >> 5) < 2 ? (o >> 5) + 1 : 2)];
  const uint32_t v = __builtin_amdgcn_alignbit(hi, lo, o & 31);
  const float off = -3.5f * d;  // exact: 13 significant bits
  half8_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t qa = (v >> (3 * i)) & 7u, qb = (v >> (3 * i + 12)) & 7u;
    r[2 * i] = (_Float16)__builtin_fmaf((float)qa, d, off);      // exact in fp32, one rounding
    r[2 * i + 1] = (_Float16)__builtin_fmaf((float)qb, d, off);
  }
  return r;
}

// Per-lane weight stream of one stage: two blocks of one row.
template <int FMT>
struct RowStage {
  uint32_t c[6];   // code bytes (Q2: 16 B in c[0..3]; Q3: 24 B)
  uint32_t sc;     // the two blocks' fp16 scales
};

template <int FMT>
STRATA_DEVICE void load_stage(RowStage<FMT>& st, const uint8_t* row_codes, const uint16_t* row_scales,
                              int blk) {
  constexpr int CB = FMT == 2 ? 8 : 12;
  const uint8_t* p = row_codes + (size_t)blk * CB;
  if constexpr (FMT == 2) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    st.c[0] = v[0]; st.c[1] = v[1]; st.c[2] = v[2]; st.c[3] = v[3];
  } else {
    const uint2* q = reinterpret_cast<const uint2*>(p);  // 8-byte aligned (blk even)
    const uint2 a = q[0], b = q[1], c = q[2];
    st.c[0] = a.x; st.c[1] = a.y; st.c[2] = b.x; st.c[3] = b.y; st.c[4] = c.x; st.c[5] = c.y;
  }
  st.sc = *reinterpret_cast<const uint32_t*>(row_scales + blk);
}

template <int FMT>
struct StageDecoder {
  Q2Tab t0, t1;
  float d0, d1;
  STRATA_DEVICE void init(const RowStage<FMT>& st) {
    if constexpr (FMT == 2) {
      t0 = q2_table((uint16_t)(st.sc & 0xFFFFu));
      t1 = q2_table((uint16_t)(st.sc >> 16));
    } else {
      d0 = f16_to_f32((uint16_t)(st.sc & 0xFFFFu));
      d1 = f16_to_f32((uint16_t)(st.sc >> 16));
    }
  }
  STRATA_DEVICE half8_t get(const RowStage<FMT>& st, int s) const {
    if constexpr (FMT == 2) {
      const u32x4_t c = {st.c[0], st.c[1], st.c[2], st.c[3]};
      return q2_decode(c, s, s < 4 ? t0 : t1);
    } else {
      return q3_decode(st.c, s, s < 4 ? d0 : d1);
    }
  }
};

// ---------------------------------------------------------------------------------------------
// Shared pieces of the two GEMMs.

struct UnitInfo {
  int expert, row_start, nrows, nfrag, slice;
};

// Maps blockIdx to a unit; false if this workgroup has no unit.
STRATA_DEVICE bool pick_unit(const Chunk* chunks, const int* n_chunks, int n_slices, UnitInfo& u) {
  const int U = *n_chunks * n_slices;
  const int per = (U + 7) >> 3;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  if (i >= per) return false;
  const int unit = xcd * per + i;
  if (unit >= U) return false;
  const Chunk ch = chunks[unit / n_slices];
  u.expert = ch.expert;
  u.row_start = ch.row_start;
  u.nrows = ch.nrows;
  u.nfrag = (ch.nrows + 31) >> 5;
  u.slice = unit % n_slices;
  return true;
}

// Stage loader of the activation tile: rows (nfrag*32) x 128 fp16 = 16 pieces of 16 B per row.
struct TileLoad {
  u32x4_t v[16];
};

STRATA_DEVICE void load_tile(TileLoad& tl, const uint16_t* __restrict__ src, const int* rows_lds,
                             int ld, int k0, int nfrag, bool gather) {
  const int npieces = nfrag * 32 * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = threadIdx.x + i * kGemmThreads;
    if (p < npieces) {
      const int r = p >> 4, c = p & 15;
      const int row = rows_lds[r];
      (void)gather;
      tl.v[i] = *reinterpret_cast<const u32x4_t*>(src + (size_t)row * ld + k0 + c * 8);
    }
  }
}

STRATA_DEVICE void store_tile(const TileLoad& tl, uint16_t* lds, int nfrag) {
  const int npieces = nfrag * 32 * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = threadIdx.x + i * kGemmThreads;
    if (p < npieces) {
      const int r = p >> 4, c = p & 15;
      *reinterpret_cast<u32x4_t*>(lds + r * kLdsRow + c * 8) = tl.v[i];
    }
  }
}

STRATA_DEVICE half8_t lds_frag(const uint16_t* lds, int f, int lane, int s) {
  const int row = f * 32 + (lane & 31);
  const int col = (lane >> 5) * 64 + s * 8;
  return *reinterpret_cast<const half8_t*>(lds + row * kLdsRow + col);
}

// ---------------------------------------------------------------------------------------------
// Up projection: A[p][n] = SiLU(x_t . W_g[n]) * (x_t . W_u[n]) for the chunk's rows p.
// Slice = 128 outputs; wave w owns outputs slice*128 + w*32 + (lane % 32), gate and up.

template <int FMT>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_up_kernel(
    const uint16_t* __restrict__ x16, const int* __restrict__ sorted_slot, int k,
    const Chunk* __restrict__ chunks, const int* __restrict__ n_chunks,
    const uint8_t* __restrict__ gate_codes, const uint8_t* __restrict__ up_codes,
    const uint16_t* __restrict__ gate_scales, const uint16_t* __restrict__ up_scales, int H, int I,
    uint16_t* __restrict__ a16) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  int* rows_lds = reinterpret_cast<int*>(smem + 2 * kLdsTile * sizeof(uint16_t));
  UnitInfo u;
  if (!pick_unit(chunks, n_chunks, I / 128, u)) return;
  constexpr int CB = FMT == 2 ? 8 : 12;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  const int nbh = H / 32;
  const int n = u.slice * 128 + wave * 32 + nl;
  const size_t grow = (size_t)u.expert * I + n;
  const uint8_t* gc = gate_codes + grow * nbh * CB;
  const uint8_t* uc = up_codes + grow * nbh * CB;
  const uint16_t* gs = gate_scales + grow * nbh;
  const uint16_t* us = up_scales + grow * nbh;

  for (int r = threadIdx.x; r < u.nfrag * 32; r += kGemmThreads)
    rows_lds[r] = sorted_slot[u.row_start + (r < u.nrows ? r : 0)] / k;
  __syncthreads();

  f32x16_t accg[kFrags], accu[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    accg[f] = f32x16_t{};
    accu[f] = f32x16_t{};
  }
  const int NK = H / kKC;
  TileLoad tl;
  RowStage<FMT> sg, su, ng, nu;
  load_tile(tl, x16, rows_lds, H, 0, u.nfrag, true);
  load_stage<FMT>(sg, gc, gs, 2 * hh);
  load_stage<FMT>(su, uc, us, 2 * hh);
  store_tile(tl, xs, u.nfrag);
  __syncthreads();
  for (int j = 0; j < NK; ++j) {
    const uint16_t* cur = xs + (j & 1) * kLdsTile;
    if (j + 1 < NK) {
      load_tile(tl, x16, rows_lds, H, (j + 1) * kKC, u.nfrag, true);
      load_stage<FMT>(ng, gc, gs, 4 * (j + 1) + 2 * hh);
      load_stage<FMT>(nu, uc, us, 4 * (j + 1) + 2 * hh);
    }
    StageDecoder<FMT> dg, du;
    dg.init(sg);
    du.init(su);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const half8_t bg = dg.get(sg, s);
      const half8_t bu = du.get(su, s);
#pragma unroll
      for (int f = 0; f < kFrags; ++f) {
        if (f < u.nfrag) {
          const half8_t a = lds_frag(cur, f, lane, s);
          accg[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bg, accg[f], 0, 0, 0);
          accu[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bu, accu[f], 0, 0, 0);
        }
      }
    }
    if (j + 1 < NK) {
      store_tile(tl, xs + ((j + 1) & 1) * kLdsTile, u.nfrag);
      sg = ng;
      su = nu;
    }
    __syncthreads();
  }
  // epilogue: lane holds column n, rows 8*(r/4) + 4*hh + r%4 of every fragment
  const int col = (n & ~7) | p8inv(n & 7);
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    if (f < u.nfrag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = f * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < u.nrows) {
          const float g = accg[f][r], up = accu[f][r];
          const float a = g / (1.0f + expf(-g)) * up;
          a16[(size_t)(u.row_start + row) * I + col] = __builtin_bit_cast(uint16_t, f32_to_f16_sat(a));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Down projection: out[slot(p)][h] = A[p] . W_d[h] for the chunk's rows p, written as bf16 in
// slot order.  Slice = 256 outputs; wave w owns h = slice*256 + w*64 + nf*32 + (lane % 32).

template <int FMT>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_down_kernel(
    const uint16_t* __restrict__ a16, const int* __restrict__ sorted_slot,
    const Chunk* __restrict__ chunks, const int* __restrict__ n_chunks,
    const uint8_t* __restrict__ down_codes, const uint16_t* __restrict__ down_scales, int H, int I,
    uint16_t* __restrict__ expert_out) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* as = reinterpret_cast<uint16_t*>(smem);
  int* rows_lds = reinterpret_cast<int*>(smem + 2 * kLdsTile * sizeof(uint16_t));
  UnitInfo u;
  if (!pick_unit(chunks, n_chunks, H / 256, u)) return;
  constexpr int CB = FMT == 2 ? 8 : 12;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  const int nbi = I / 32;
  const int h0 = u.slice * 256 + wave * 64 + nl;
  const size_t r0 = (size_t)u.expert * H + h0, r1 = r0 + 32;
  const uint8_t* c0 = down_codes + r0 * nbi * CB;
  const uint8_t* c1 = down_codes + r1 * nbi * CB;
  const uint16_t* s0 = down_scales + r0 * nbi;
  const uint16_t* s1 = down_scales + r1 * nbi;

  for (int r = threadIdx.x; r < u.nfrag * 32; r += kGemmThreads)
    rows_lds[r] = u.row_start + (r < u.nrows ? r : 0);
  __syncthreads();

  f32x16_t acc0[kFrags], acc1[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    acc0[f] = f32x16_t{};
    acc1[f] = f32x16_t{};
  }
  const int NK = I / kKC;
  TileLoad tl;
  RowStage<FMT> st0, st1, nx0, nx1;
  load_tile(tl, a16, rows_lds, I, 0, u.nfrag, false);
  load_stage<FMT>(st0, c0, s0, 2 * hh);
  load_stage<FMT>(st1, c1, s1, 2 * hh);
  store_tile(tl, as, u.nfrag);
  __syncthreads();
  for (int j = 0; j < NK; ++j) {
    const uint16_t* cur = as + (j & 1) * kLdsTile;
    if (j + 1 < NK) {
      load_tile(tl, a16, rows_lds, I, (j + 1) * kKC, u.nfrag, false);
      load_stage<FMT>(nx0, c0, s0, 4 * (j + 1) + 2 * hh);
      load_stage<FMT>(nx1, c1, s1, 4 * (j + 1) + 2 * hh);
    }
    StageDecoder<FMT> d0, d1;
    d0.init(st0);
    d1.init(st1);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const half8_t b0 = d0.get(st0, s);
      const half8_t b1 = d1.get(st1, s);
#pragma unroll
      for (int f = 0; f < kFrags; ++f) {
        if (f < u.nfrag) {
          const half8_t a = lds_frag(cur, f, lane, s);
          acc0[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc0[f], 0, 0, 0);
          acc1[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc1[f], 0, 0, 0);
        }
      }
    }
    if (j + 1 < NK) {
      store_tile(tl, as + ((j + 1) & 1) * kLdsTile, u.nfrag);
      st0 = nx0;
      st1 = nx1;
    }
    __syncthreads();
  }
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    if (f < u.nfrag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = f * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < u.nrows) {
          const size_t slot = (size_t)sorted_slot[u.row_start + row];
          expert_out[slot * H + h0] = f32_to_bf16(acc0[f][r]);
          expert_out[slot * H + h0 + 32] = f32_to_bf16(acc1[f][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// x bf16 -> fp16 in P8 order (one thread per 8 values).

__global__ void x_to_f16_kernel(const uint16_t* __restrict__ x, size_t n8, uint16_t* __restrict__ x16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u32x4_t v = reinterpret_cast<const u32x4_t*>(x)[i];
  uint16_t in[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    in[2 * m] = (uint16_t)(v[m] & 0xFFFFu);
    in[2 * m + 1] = (uint16_t)(v[m] >> 16);
  }
  constexpr int P8[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  u32x4_t o;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, f32_to_f16_sat(bf16_to_f32(in[P8[2 * m]])));
    const uint32_t hi = __builtin_bit_cast(uint16_t, f32_to_f16_sat(bf16_to_f32(in[P8[2 * m + 1]])));
    o[m] = lo | (hi << 16);
  }
  reinterpret_cast<u32x4_t*>(x16)[i] = o;
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t][h] (+)= sum_j w[t][j] * out[t*k + j][h], j ascending (one thread per 8 h).

__global__ void combine_kernel(const uint16_t* __restrict__ out, const float* __restrict__ w, int T,
                               int k, int H, float* __restrict__ y, int accumulate) {
  const int h8 = H / 8;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * h8) return;
  const int t = (int)(i / h8), c = (int)(i % h8);
  float acc[8];
  if (accumulate) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(y + (size_t)t * H + c * 8)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(y + (size_t)t * H + c * 8)[1];
#pragma unroll
    for (int m = 0; m < 4; ++m) { acc[m] = a[m]; acc[m + 4] = b[m]; }
  }
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(out + ((size_t)t * k + j) * H + c * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[2 * m] = __builtin_fmaf(wj, __uint_as_float(v[m] << 16), s[2 * m]);
      s[2 * m + 1] = __builtin_fmaf(wj, __uint_as_float(v[m] & 0xFFFF0000u), s[2 * m + 1]);
    }
  }
  f32x4_t o0, o1;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    o0[m] = accumulate ? acc[m] + s[m] : s[m];
    o1[m] = accumulate ? acc[m + 4] + s[m + 4] : s[m + 4];
  }
  reinterpret_cast<f32x4_t*>(y + (size_t)t * H + c * 8)[0] = o0;
  reinterpret_cast<f32x4_t*>(y + (size_t)t * H + c * 8)[1] = o1;
}

// ---------------------------------------------------------------------------------------------
// RMSNorm (unit gain): one workgroup of 256 threads per row.

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int H, float eps,
                                                      uint16_t* __restrict__ x) {
  __shared__ float part[4];
  const float* row = h + (size_t)blockIdx.x * H;
  float ss = 0.0f;
  for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
    ss = __builtin_fmaf(v[0], v[0], ss);
    ss = __builtin_fmaf(v[1], v[1], ss);
    ss = __builtin_fmaf(v[2], v[2], ss);
    ss = __builtin_fmaf(v[3], v[3], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* xr = x + (size_t)blockIdx.x * H;
  for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
    const uint32_t lo = f32_to_bf16(v[0] * inv) | ((uint32_t)f32_to_bf16(v[1] * inv) << 16);
    const uint32_t hi = f32_to_bf16(v[2] * inv) | ((uint32_t)f32_to_bf16(v[3] * inv) << 16);
    *reinterpret_cast<uint2*>(xr + i) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------------------------
// Launchers

static int grid_for_units(int64_t max_units) { return (int)(8 * ((max_units + 7) / 8)); }

// The GEMM kernels use more than 64 KB of dynamic LDS; allow it once per process.
static void allow_big_lds() {
  static std::once_flag once;
  std::call_once(once, [] {
    const void* ks[4] = {reinterpret_cast<const void*>(ffn_up_kernel<2>),
                         reinterpret_cast<const void*>(ffn_up_kernel<3>),
                         reinterpret_cast<const void*>(ffn_down_kernel<2>),
                         reinterpret_cast<const void*>(ffn_down_kernel<3>)};
    for (const void* k : ks)
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
  });
}

hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, hipStream_t s) {
  const size_t n8 = (size_t)T * H / 8;
  x_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, x16);
  return hipGetLastError();
}

hipError_t launch_ffn_up(int fmt, const uint16_t* x16, const int* sorted_slot, int k,
                         const Chunk* chunks, const int* n_chunks, int max_chunks_,
                         const void* gate_codes, const void* up_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, int E, int H, int I, uint16_t* a16,
                         hipStream_t s) {
  (void)E;
  const int grid = grid_for_units((int64_t)max_chunks_ * (I / 128));
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  if (fmt == 2) {
    allow_big_lds();
    ffn_up_kernel<2><<<grid, kGemmThreads, kGemmLds, s>>>(x16, sorted_slot, k, chunks, n_chunks, gc,
                                                          uc, gate_scales, up_scales, H, I, a16);
  } else {
    allow_big_lds();
    ffn_up_kernel<3><<<grid, kGemmThreads, kGemmLds, s>>>(x16, sorted_slot, k, chunks, n_chunks, gc,
                                                          uc, gate_scales, up_scales, H, I, a16);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(int fmt, const uint16_t* a16, const int* sorted_slot,
                           const Chunk* chunks, const int* n_chunks, int max_chunks_,
                           const void* down_codes, const uint16_t* down_scales, int E, int H,
                           int I, uint16_t* expert_out, hipStream_t s) {
  (void)E;
  const int grid = grid_for_units((int64_t)max_chunks_ * (H / 256));
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  if (fmt == 2) {
    allow_big_lds();
    ffn_down_kernel<2><<<grid, kGemmThreads, kGemmLds, s>>>(a16, sorted_slot, chunks, n_chunks, dc,
                                                            down_scales, H, I, expert_out);
  } else {
    allow_big_lds();
    ffn_down_kernel<3><<<grid, kGemmThreads, kGemmLds, s>>>(a16, sorted_slot, chunks, n_chunks, dc,
                                                            down_scales, H, I, expert_out);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* expert_out, const float* w, int T, int k, int H, float* y,
                          int accumulate, hipStream_t s) {
  const size_t n = (size_t)T * (H / 8);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(expert_out, w, T, k, H, y, accumulate);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, int T, int H, float eps, uint16_t* x, hipStream_t s) {
  rmsnorm_kernel<<<T, 256, 0, s>>>(h, H, eps, x);
  return hipGetLastError();
}

}  // namespace strata
