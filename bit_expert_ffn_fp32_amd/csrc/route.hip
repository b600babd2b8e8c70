// Router: per-token top-k over fp32 logits, one 64-lane wave per token.
//
// The pages route each token to 10 of a layer's 512 experts with the routers on the GPU
// ("Strata vs Llama.cpp vs vLLM", transcript at 08:23 and 09:28); they give no formula.  Here:
// softmax over all logits, keep the k largest, renormalise.  Softmax is monotone, so the choice is
// made on the logits themselves: k rounds of a wave-wide arg-max in which expert a beats b iff
// l_a > l_b, or l_a == l_b and a < b.  The kept weights are exp(l_j - l_0) / sum_i exp(l_i - l_0).
//
// Lane l holds experts l, l + 64, l + 128, ... so every load of a token's row is coalesced.
#include "common.hpp"
#include "kernels.hpp"

namespace strata {

template <int NPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[NPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
    if (e >= E) taken |= 1u << i;
  }
  float my_v = 0.0f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      const bool free_ = !((taken >> i) & 1u);
      // within a lane e grows with i, so a strict '>' keeps the lower index on ties
      if (free_ && (bi == 0x7FFFFFFF || v[i] > bv)) { bv = v[i]; bi = e; }
    }
    // lanes with nothing left must lose every comparison
    if (bi == 0x7FFFFFFF) bv = -__builtin_inff();
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) { my_v = bv; my_i = bi; }
  }
  const float top = __shfl(my_v, 0);
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  const float den = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_i;
    w[(size_t)t * k + lane] = ex / den;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t s) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  if (E <= 64) route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128) route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256) route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 512) route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace strata
