// Router: per-token top-k over fp32 logits, one 64-lane wave per token.
//
// The pages route each token to 10 of a layer's 512 experts with the routers on the GPU
// ("Strata vs Llama.cpp vs vLLM", transcript at 08:23 and 09:28); they give no formula.  Here:
// softmax over all logits, keep the k largest, renormalise.  Softmax is monotone, so the choice is
// made on the logits themselves: the k largest under the order in which expert a beats b iff
// l_a > l_b, or l_a == l_b and a < b.  The kept weights are exp(l_j - l_0) / sum_i exp(l_i - l_0).
//
// Lane l holds experts l, l + 64, l + 128, ... so every load of a token's row is coalesced.  Each
// lane sorts its own entries once (largest first); the k-th largest lane head bounds the selection
// from below, the few entries above it are ranked against each other in LDS (k rounds of a
// wave-wide arg-max where more than 64 pass), the selection the decode kernel runs too.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace strata {

constexpr int kRouteWaves = 4;  // tokens (waves) per workgroup

template <int NPL>
__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int* __restrict__ ids,
                                                    float* __restrict__ w) {
  __shared__ __align__(16) uint64_t sel[kRouteWaves][80];
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  TokenKeys<NPL> tk;
  load_token_logits<NPL>(logits + (size_t)t * E, E, tk);
  select_token_wave<NPL>(tk, E, k, ids + (size_t)t * k, w + (size_t)t * k, sel[threadIdx.x >> 6]);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t s) {
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves), block(64 * kRouteWaves);
  if (E <= 64) route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128) route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256) route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 512) route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace strata
