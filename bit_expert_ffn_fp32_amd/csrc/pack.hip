// Weight repack: row-major block-quantized matrices -> the tiled device layout read by the GEMM
// and decode kernels.
//
// A matrix of R rows (a multiple of 4) and reduction length K (a multiple of 64) is cut into
// 4-row x 64-index tiles (two 32-weight blocks per row); tile (g, kt) holds rows 4 g .. 4 g + 3,
// each row's two blocks' codes consecutive (16 or 24 bytes), and its scales likewise (two fp16 per
// row).  Tiles are ordered g-major, kt-minor.  So a 4-row group's successive 64-index stages are
// contiguous (what a decode wave streams: 4 rows x 16 stages = one contiguous 1 KB), and one stage
// of 64 rows is 16 pieces of 64 (or 96) bytes (what a GEMM stage copies), instead of 64 separate
// 16-byte pieces in the row-major layout.
#include "common.hpp"
#include "kernels.hpp"
#include "strata_moe.h"

namespace strata {

// One thread per (matrix, row, tile-stage), in tiled order so the stores are contiguous.
template <int CB>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int R, int K,
                                                   size_t n, uint8_t* __restrict__ tcodes,
                                                   uint16_t* __restrict__ tscales) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int nkt = K / 64;
  const int r = (int)(i & 3);
  const size_t rest = i >> 2;                  // (row group, tile-stage)
  const int kt = (int)(rest % nkt);
  const size_t row = rest / nkt * 4 + r;       // global row over all matrices
  const uint8_t* src = codes + row * (size_t)(K / 32) * CB + (size_t)kt * 2 * CB;
  uint8_t* dst = tcodes + i * 2 * CB;
  if constexpr (CB == 8) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else {
#pragma unroll
    for (int q = 0; q < 3; ++q)
      reinterpret_cast<uint2*>(dst)[q] = reinterpret_cast<const uint2*>(src)[q];
  }
  *reinterpret_cast<uint32_t*>(tscales + i * 2) =
      *reinterpret_cast<const uint32_t*>(scales + row * (size_t)(K / 32) + (size_t)kt * 2);
}

hipError_t launch_pack(int fmt, int n_mat, int R, int K, const void* codes, const uint16_t* scales,
                       void* tcodes, uint16_t* tscales, hipStream_t s) {
  const size_t n = (size_t)n_mat * R * (K / 64);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (fmt == 2)
    pack_kernel<8><<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(codes), scales, R, K, n,
                                        static_cast<uint8_t*>(tcodes), tscales);
  else
    pack_kernel<12><<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(codes), scales, R, K, n,
                                         static_cast<uint8_t*>(tcodes), tscales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Range statistics per expert (one workgroup per expert): for gate and up, the largest |d| and
// the largest row 2-norm; for down, the largest |d|.  A row's squared norm is the sum over its
// blocks of d^2 * sum_i (q_i - c0)^2, formed in fp64 (a one-time load step); sum_i (q_i - c0)^2
// is a quarter of the integer sum of (2 q_i - 2 c0)^2.

template <int CB>
STRATA_DEVICE int code_sq4(const uint8_t* blk) {
  // 4 * sum over the block of (q - c0)^2, exactly
  int sum = 0;
  if constexpr (CB == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(blk);
    for (int i = 0; i < 32; ++i) {
      const int q = (int)(((i < 16 ? v.x : v.y) >> (2 * (i & 15))) & 3u);
      sum += (2 * q - 3) * (2 * q - 3);
    }
  } else {
    const uint32_t w0 = reinterpret_cast<const uint32_t*>(blk)[0];
    const uint32_t w1 = reinterpret_cast<const uint32_t*>(blk)[1];
    const uint32_t w2 = reinterpret_cast<const uint32_t*>(blk)[2];
    const uint64_t lo = (uint64_t)w0 | ((uint64_t)w1 << 32);
    for (int i = 0; i < 32; ++i) {
      const int bit = 3 * i;
      uint32_t q;
      if (bit + 3 <= 64) q = (uint32_t)(lo >> bit) & 7u;
      else if (bit >= 64) q = (w2 >> (bit - 64)) & 7u;
      else q = (uint32_t)((lo >> bit) | ((uint64_t)w2 << (64 - bit))) & 7u;
      sum += (2 * (int)q - 7) * (2 * (int)q - 7);
    }
  }
  return sum;
}

// Largest |d| and largest row norm of one tiled matrix of R rows x K (this expert's part).
template <int CB>
STRATA_DEVICE void matrix_range(const uint8_t* codes, const uint16_t* scales, int R, int K,
                                bool norms, double* red, double& dmax, double& nmax) {
  const int nkt = K / 64, nb = K / 32;
  double dm = 0.0, nm = 0.0;
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    double ss = 0.0;
    for (int b = 0; b < nb; ++b) {
      const size_t idx = (((size_t)(r >> 2) * nkt + (b >> 1)) * 4 + (r & 3)) * 2 + (b & 1);
      const double d = (double)__builtin_bit_cast(_Float16, scales[idx]);
      dm = fmax(dm, fabs(d));
      if (norms) ss += d * d * (0.25 * (double)code_sq4<CB>(codes + idx * CB));
    }
    nm = fmax(nm, ss);
  }
  red[threadIdx.x] = dm;
  red[blockDim.x + threadIdx.x] = nm;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + o]);
      red[blockDim.x + threadIdx.x] = fmax(red[blockDim.x + threadIdx.x], red[blockDim.x + threadIdx.x + o]);
    }
    __syncthreads();
  }
  dmax = red[0];
  nmax = sqrt(red[blockDim.x]);
  __syncthreads();
}

// Shift s with dmax * c0max * 2^s in [2^14, 2^15) (0 for an all-zero matrix), at most smax.
STRATA_DEVICE int range_shift(double dmax, double c0max, int smax) {
  const double m = dmax * c0max;
  if (!(m > 0.0)) return 0;
  int e;
  (void)frexp(m, &e);  // m in [2^(e-1), 2^e)
  return 15 - e < smax ? 15 - e : smax;
}

template <int CB>
__global__ __launch_bounds__(256) void weight_stats_kernel(
    const uint8_t* __restrict__ gc, const uint8_t* __restrict__ uc, const uint8_t* __restrict__ dc,
    const uint16_t* __restrict__ gs, const uint16_t* __restrict__ us,
    const uint16_t* __restrict__ ds, int H, int I, strata_moe_expert_stats* __restrict__ out) {
  __shared__ double red[512];
  const int e = blockIdx.x;
  const double c0max = CB == 8 ? 1.5 : 3.5;
  const size_t gu_blocks = (size_t)I * (H / 32), d_blocks = (size_t)H * (I / 32);
  double dg, ng, du, nu, dd, nd;
  matrix_range<CB>(gc + e * gu_blocks * CB, gs + e * gu_blocks, I, H, true, red, dg, ng);
  matrix_range<CB>(uc + e * gu_blocks * CB, us + e * gu_blocks, I, H, true, red, du, nu);
  matrix_range<CB>(dc + e * d_blocks * CB, ds + e * d_blocks, H, I, false, red, dd, nd);
  if (threadIdx.x == 0) {
    // 2-bit: the GEMM scales its code-offset constants (exact in fp16 up to 2^15 * 1.5)
    const int smax = CB == 8 ? 15 : 64;
    const int sg = range_shift(dg, c0max, smax), su = range_shift(du, c0max, smax),
              sd = range_shift(dd, c0max, smax);
    // fp16 rounding of the shifted weights grows a norm by at most 2^-11; 2^-9 of margin
    const double n = ldexp(ng, sg) * ldexp(nu, su) * (1.0 + 0x1p-9);
    out[e] = strata_moe_expert_stats{sg, su, sd, (float)n};
  }
}

hipError_t launch_weight_stats(int fmt, int E, int H, int I, const void* gate_codes,
                               const void* up_codes, const void* down_codes,
                               const uint16_t* gate_scales, const uint16_t* up_scales,
                               const uint16_t* down_scales, strata_moe_expert_stats* stats,
                               hipStream_t s) {
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  if (fmt == 2)
    weight_stats_kernel<8><<<E, 256, 0, s>>>(gc, uc, dc, gate_scales, up_scales, down_scales, H, I, stats);
  else
    weight_stats_kernel<12><<<E, 256, 0, s>>>(gc, uc, dc, gate_scales, up_scales, down_scales, H, I, stats);
  return hipGetLastError();
}

}  // namespace strata
