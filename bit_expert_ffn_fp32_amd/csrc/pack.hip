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

}  // namespace strata
