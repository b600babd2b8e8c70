// Expert usage statistics: per-expert slot counts accumulated over calls, and the hotness order.
//
// The pages' engine keeps a running distribution of how often each expert is used and keeps the
// most-used ones close to the compute (video transcript on unbiasedbob.com, 7:47 to 7:58; "Strata
// - the details", How it works / memory tiers).  With every expert resident in HBM there is no
// cache to fill, but the statistic itself is cheap to keep and export: usage[e] += the number of
// (token, slot) pairs routed to e, and the order of experts by usage (ties to the lower index).
#include "common.hpp"
#include "kernels.hpp"

namespace strata {

constexpr int kUsageThreads = 1024;
constexpr int kUsageSlotsPerThread = 8;

// One LDS histogram per workgroup over its slice of slots, then one 64-bit atomic add per
// non-empty bin: integer adds, so the result does not depend on their order.
__global__ __launch_bounds__(kUsageThreads) void usage_update_kernel(const int* __restrict__ ids,
                                                                     int64_t S, int E,
                                                                     unsigned long long* usage) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E; e += kUsageThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kUsageThreads * kUsageSlotsPerThread;
#pragma unroll
  for (int i = 0; i < kUsageSlotsPerThread; ++i) {
    const int64_t s = base + (int64_t)i * kUsageThreads + threadIdx.x;
    if (s < S) {
      const int e = ids[s];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kUsageThreads)
    if (hist[e]) atomicAdd(usage + e, (unsigned long long)hist[e]);
}

// One workgroup: thread e counts the experts ranked before it (more uses, or as many and a lower
// index) and writes itself at that rank.
__global__ __launch_bounds__(kUsageThreads) void usage_rank_kernel(const unsigned long long* usage,
                                                                   int E, int* order) {
  __shared__ unsigned long long u[1024];
  const int e = threadIdx.x;
  if (e < E) u[e] = usage[e];
  __syncthreads();
  if (e >= E) return;
  const unsigned long long me = u[e];
  int rank = 0;
  for (int j = 0; j < E; ++j) {
    const unsigned long long v = u[j];
    rank += (v > me) || (v == me && j < e);
  }
  order[rank] = e;
}

hipError_t launch_usage_update(const int* ids, int64_t S, int E, uint64_t* usage, hipStream_t s) {
  const int64_t per_block = (int64_t)kUsageThreads * kUsageSlotsPerThread;
  const int grid = (int)((S + per_block - 1) / per_block);
  hipLaunchKernelGGL(usage_update_kernel, dim3(grid), dim3(kUsageThreads), 0, s, ids, S, E,
                     reinterpret_cast<unsigned long long*>(usage));
  return hipGetLastError();
}

hipError_t launch_usage_rank(const uint64_t* usage, int E, int* order, hipStream_t s) {
  hipLaunchKernelGGL(usage_rank_kernel, dim3(1), dim3(kUsageThreads), 0, s,
                     reinterpret_cast<const unsigned long long*>(usage), E, order);
  return hipGetLastError();
}

}  // namespace strata
