// Permute: group the T*k (token, slot) pairs by expert with a stable counting sort.
//
// The pages imply per-expert work lists (each expert's matrix multiply runs over the tokens
// routed to it: "Two-Day Port, 8x Faster Prefill: Strata Engine Benchmarked", Where Strata Is
// Fast) but print no algorithm.  Slot s = t*k + j; expert e's segment of the sorted order lists
// its slots in ascending s.
//
// Three kernels, all integer work:
//  1. count:   one workgroup per tile of kPermTile slots builds the tile's expert histogram
//              (LDS integer atomics: the result is order independent).
//  2. scan:    one workgroup turns the histograms into counts, offsets (exclusive prefix sum)
//              and each tile's starting position per expert; it also cuts every expert's segment
//              into GEMM chunks of at most kChunkRows rows, balanced in 32-row fragments.
//  3. scatter: each tile ranks its slots stably: in rounds of 256 slots, a slot's rank is the
//              number of equal ids in earlier lanes of its wave (an LDS broadcast loop), plus the
//              counts of earlier waves of the round, plus the tile's running count.
#include "common.hpp"
#include "kernels.hpp"

namespace strata {

constexpr int kPermThreads = 256;

__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(const int* __restrict__ ids,
                                                                      int S, int E,
                                                                      int* __restrict__ hist) {
  extern __shared__ int h[];
  for (int e = threadIdx.x; e < E; e += kPermThreads) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermTile;
#pragma unroll
  for (int r = 0; r < kPermTile / kPermThreads; ++r) {
    const int s = base + r * kPermThreads + threadIdx.x;
    if (s < S) {
      const int id = ids[s];
      if ((unsigned)id < (unsigned)E) atomicAdd(&h[id], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) hist[(size_t)blockIdx.x * E + e] = h[e];
}

// Exclusive prefix sum over the block (blockDim.x = 1024 = 16 waves); returns the block total.
__device__ int block_exclusive_scan(int v, int* lds16, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) lds16[wv] = inc;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    const int t = lds16[i];
    if (i < wv) wbase += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return wbase + inc - v;
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(
    const int* __restrict__ hist, int ntiles, int E, int* __restrict__ tile_base,
    int* __restrict__ counts, int* __restrict__ offsets, Chunk* __restrict__ chunks,
    int* __restrict__ n_chunks) {
  __shared__ int lds16[16];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    int t = 0;
    for (; t + 8 <= ntiles; t += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(size_t)(t + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt += v[u];
    }
    for (; t < ntiles; ++t) cnt += hist[(size_t)t * E + e];
  }
  int total;
  const int off = block_exclusive_scan(e < E ? cnt : 0, lds16, total);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + cnt;
    int run = off;
    int t = 0;
    for (; t + 8 <= ntiles; t += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(size_t)(t + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tile_base[(size_t)(t + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; t < ntiles; ++t) {
      tile_base[(size_t)t * E + e] = run;
      run += hist[(size_t)t * E + e];
    }
  }
  if (chunks == nullptr) return;
  // GEMM chunks: ceil(cnt / kChunkRows) per expert, fragments of 32 rows spread evenly.
  const int nfrag = (cnt + 31) / 32;
  const int nch = (nfrag + (kChunkRows / 32) - 1) / (kChunkRows / 32);
  int ctotal;
  const int cbase = block_exclusive_scan(e < E ? nch : 0, lds16, ctotal);
  if (e < E && nch > 0) {
    const int fb = nfrag / nch, extra = nfrag % nch;
    int row = off, frag_used = 0;
    for (int c = 0; c < nch; ++c) {
      const int nf = fb + (c < extra ? 1 : 0);
      const int rows = min(nf * 32, cnt - frag_used * 32);
      chunks[cbase + c] = Chunk{e, row, rows, 0};
      row += rows;
      frag_used += nf;
    }
  }
  if (e == 0) *n_chunks = ctotal;
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int* __restrict__ ids, int S, int E, const int* __restrict__ tile_base,
    int* __restrict__ sorted_slot, int* __restrict__ slot_pos) {
  extern __shared__ int lds[];
  int* cnt = lds;                 // [E] running position per expert
  int* wc = lds + E;              // [4][E] per-wave counts of the current round
  int* ids_l = lds + 5 * E;       // [256] ids of the current round
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += kPermThreads) {
    cnt[e] = tile_base[(size_t)blockIdx.x * E + e];
    wc[e] = wc[E + e] = wc[2 * E + e] = wc[3 * E + e] = 0;
  }
  const int base = blockIdx.x * kPermTile;
  for (int r = 0; r < kPermTile / kPermThreads; ++r) {
    const int s = base + r * kPermThreads + tid;
    const int id0 = s < S ? ids[s] : -1;
    const bool valid = (unsigned)id0 < (unsigned)E;  // out-of-range ids are skipped
    const int id = valid ? id0 : -1;
    ids_l[tid] = id;
    __syncthreads();
    int rank = 0;
    bool last = true;
    const int* wids = ids_l + wv * 64;
    for (int i = 0; i < 64; ++i) {
      const int o = wids[i];
      rank += (i < lane && o == id) ? 1 : 0;
      last = last && !(i > lane && o == id);
    }
    if (valid && last) wc[wv * E + id] = rank + 1;
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w2 = 0; w2 < wv; ++w2) before += wc[w2 * E + id];
      const int pos = cnt[id] + before + rank;
      sorted_slot[pos] = s;
      slot_pos[s] = pos;
    }
    __syncthreads();
    if (valid && last) {
      atomicAdd(&cnt[id], rank + 1);
      wc[wv * E + id] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_permute(const int* ids, int T, int E, int k, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, int* tile_hist, int* tile_base,
                          Chunk* chunks, int* n_chunks, hipStream_t s) {
  const int S = T * k;
  const int ntiles = (S + kPermTile - 1) / kPermTile;
  permute_count_kernel<<<ntiles, kPermThreads, E * sizeof(int), s>>>(ids, S, E, tile_hist);
  permute_scan_kernel<<<1, 1024, 0, s>>>(tile_hist, ntiles, E, tile_base, counts, offsets, chunks,
                                         n_chunks);
  permute_scatter_kernel<<<ntiles, kPermThreads, (5 * E + kPermThreads) * sizeof(int), s>>>(
      ids, S, E, tile_base, sorted_slot, slot_pos);
  return hipGetLastError();
}

}  // namespace strata
