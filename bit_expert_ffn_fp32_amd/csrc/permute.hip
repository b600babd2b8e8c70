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
//  3. scatter: each tile ranks its slots stably in one round of 1024 threads: a slot's rank is the
//              number of equal ids in earlier lanes of its wave (an LDS broadcast loop), plus the
//              counts of the earlier waves, plus the tile's starting position for its expert.
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

// hist[t][e] summed over the tiles [t0, t1) of one expert, 16 loads in flight at a time.
__device__ int tile_sum(const int* __restrict__ hist, int E, int e, int t0, int t1) {
  int acc = 0;
  for (int t = t0; t < t1; t += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = t + u < t1 ? hist[(size_t)(t + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += v[u];
  }
  return acc;
}

// P = 1024 / E' threads per expert (E' = E rounded up to a power of two): part q of expert e
// handles tiles [q nt / P, (q+1) nt / P), so the loads of a long tile list are spread over P
// threads.
__global__ __launch_bounds__(1024) void permute_scan_kernel(
    const int* __restrict__ hist, int ntiles, int E, int P, int* __restrict__ tile_base,
    int* __restrict__ counts, int* __restrict__ offsets, Chunk* __restrict__ chunks,
    int* __restrict__ n_chunks) {
  __shared__ int lds16[16];
  __shared__ int psum[1024];  // [part][e]
  const int Ep = 1024 / P;    // threads of one part (>= E)
  const int q = threadIdx.x / Ep, e = threadIdx.x % Ep;
  const bool mine = e < E;
  const int t0 = (int)((int64_t)ntiles * q / P), t1 = (int)((int64_t)ntiles * (q + 1) / P);
  const int part = mine ? tile_sum(hist, E, e, t0, t1) : 0;
  psum[threadIdx.x] = part;
  __syncthreads();
  int cnt = 0, before = 0;  // the expert's count, and the parts before this one
  if (mine) {
    for (int r = 0; r < P; ++r) {
      const int v = psum[r * Ep + e];
      cnt += v;
      before += r < q ? v : 0;
    }
  }
  int total;
  const int off = block_exclusive_scan(q == 0 && mine ? cnt : 0, lds16, total);
  __shared__ int off_e[1024];
  if (q == 0) off_e[e] = off;
  __syncthreads();
  if (mine) {
    const int o = off_e[e];
    if (q == 0) {
      counts[e] = cnt;
      offsets[e] = o;
      if (e == E - 1) offsets[E] = o + cnt;
    }
    int run = o + before;
    for (int t = t0; t < t1; t += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = t + u < t1 ? hist[(size_t)(t + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (t + u < t1) tile_base[(size_t)(t + u) * E + e] = run;
        run += v[u];
      }
    }
  }
  if (chunks == nullptr) return;
  // GEMM chunks: ceil(cnt / kChunkRows) per expert, fragments of 32 rows spread evenly.
  const int nfrag = (cnt + 31) / 32;
  const int nch = (nfrag + (kChunkRows / 32) - 1) / (kChunkRows / 32);
  int ctotal;
  const int cbase = block_exclusive_scan(q == 0 && mine ? nch : 0, lds16, ctotal);
  if (q == 0 && mine && nch > 0) {
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
  if (threadIdx.x == 0) *n_chunks = ctotal;
}

// One workgroup of 1024 threads (16 waves) per tile of kPermTile = 1024 slots, in one round: a
// slot's rank is the number of equal ids in earlier lanes of its wave (an LDS broadcast loop)
// plus the counts of the earlier waves, plus the tile's starting position for its expert.
constexpr int kScatterThreads = 1024;
constexpr int kScatterWaves = kScatterThreads / 64;
static_assert(kPermTile == kScatterThreads, "one slot per thread");

__global__ __launch_bounds__(kScatterThreads) void permute_scatter_kernel(
    const int* __restrict__ ids, int S, int E, const int* __restrict__ tile_base,
    int* __restrict__ sorted_slot, int* __restrict__ slot_pos) {
  extern __shared__ int lds[];
  int* ids_l = lds;                                               // [1024]
  uint8_t* wc = reinterpret_cast<uint8_t*>(lds + kScatterThreads);  // [16][E] per-wave counts (<= 64)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < kScatterWaves * E / 4; i += kScatterThreads) reinterpret_cast<int*>(wc)[i] = 0;
  const int s = blockIdx.x * kPermTile + tid;
  const int id0 = s < S ? ids[s] : -1;
  const bool valid = (unsigned)id0 < (unsigned)E;  // out-of-range ids are skipped
  const int id = valid ? id0 : -1;
  const int base = valid ? tile_base[(size_t)blockIdx.x * E + id] : 0;
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
  if (valid && last) wc[wv * E + id] = (uint8_t)(rank + 1);
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w2 = 0; w2 < wv; ++w2) before += wc[w2 * E + id];
    const int pos = base + before + rank;
    sorted_slot[pos] = s;
    slot_pos[s] = pos;
  }
}

hipError_t launch_permute(const int* ids, int T, int E, int k, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, int* tile_hist, int* tile_base,
                          Chunk* chunks, int* n_chunks, hipStream_t s) {
  const int S = T * k;
  const int ntiles = (S + kPermTile - 1) / kPermTile;
  permute_count_kernel<<<ntiles, kPermThreads, E * sizeof(int), s>>>(ids, S, E, tile_hist);
  int Ep = 1;
  while (Ep < E) Ep <<= 1;  // E <= 1024
  permute_scan_kernel<<<1, 1024, 0, s>>>(tile_hist, ntiles, E, 1024 / Ep, tile_base, counts,
                                         offsets, chunks, n_chunks);
  const size_t scatter_lds = kScatterThreads * sizeof(int) + ((size_t)kScatterWaves * E + 3) / 4 * 4;
  permute_scatter_kernel<<<ntiles, kScatterThreads, scatter_lds, s>>>(ids, S, E, tile_base,
                                                                      sorted_slot, slot_pos);
  return hipGetLastError();
}

}  // namespace strata
