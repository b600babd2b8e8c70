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
//              into the GEMM chunk list (one chunk per expert of at most kChunkRowsSmall rows, those
//              of at most kSkinnyRows first; chunks of up to kChunkRows rows for the others,
//              balanced in 32-row fragments).
//  3. scatter: each tile ranks its slots stably in one round of 1024 threads: a slot's rank is the
//              number of equal ids in earlier lanes of its wave (an LDS broadcast loop), plus the
//              counts of the earlier waves, plus the tile's starting position for its expert.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

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

// Exclusive prefix sums over the block (1024 threads = 16 waves) of N values a thread at once,
// and their block totals: a DPP scan within each wave, then every wave scans the 16 wave totals
// from LDS (lds: 16 N ints).  Independent scans share the two barriers.
template <int N>
__device__ void block_scan(const int (&v)[N], int (&excl)[N], int (&total)[N], int* lds) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int inc[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    inc[n] = wave_scan_dpp(v[n]);
    if (lane == 63) lds[16 * n + wv] = inc[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int t = lane < 16 ? lds[16 * n + lane] : 0;
    const int ti = wave_scan_dpp(t);
    excl[n] = __builtin_amdgcn_readlane(ti - t, wv) + inc[n] - v[n];
    total[n] = __builtin_amdgcn_readlane(ti, 15);
  }
  __syncthreads();  // (lds is reused by the next scan)
}

// The two-part GEMM chunk list (see ChunkList), built by a whole 1024-thread workgroup; a thread
// with mine holds expert e, its rows at sorted positions [off, off + cnt); nsmall: the number of
// experts with small_chunks_of(cnt, cl.small_rows) (the caller's scan).  The small part is used
// only when at least cl.min_small experts qualify for it; within it the chunks of at most
// kSkinnyRows rows come first (with the experts of up to 2 kSkinnyRows rows split in two when at
// most kSkinnySplitMax of them exist), each group in expert order.  lds: 48 ints.
__device__ void build_chunk_list(bool mine, int e, int off, int cnt, const ChunkList& cl,
                                 int nsmall, int* lds) {
  const int sr = nsmall >= cl.min_small ? cl.small_rows : 0;
  const int small = mine ? small_chunks_of(cnt, sr) : 0;
  // small-part experts of more than kSkinnyRows rows
  const int vw[1] = {small && cnt > kSkinnyRows ? 1 : 0};
  int ew[1], nwide[1];
  block_scan<1>(vw, ew, nwide, lds);
  // skinny chunks of this expert: one, two halves of a split one, or none
  const int nsk = !small ? 0 : cnt <= kSkinnyRows ? 1 : nwide[0] <= kSkinnySplitMax ? 2 : 0;
  // positions in the skinny list, in the rest of the small part and in the large part
  const int v[3] = {nsk, small && !nsk ? 1 : 0, mine ? large_chunks_of(cnt, sr) : 0};
  int b[3], n[3];
  block_scan<3>(v, b, n, lds);
  const int nskinny = n[0];
  if (nsk == 2) {
    cl.chunks[b[0]] = Chunk{e, off, kSkinnyRows, 0};
    cl.chunks[b[0] + 1] = Chunk{e, off + kSkinnyRows, cnt - kSkinnyRows, 0};
  } else if (mine) {
    write_expert_chunks(e, off, cnt, sr, cl.chunks, nsk ? b[0] : nskinny + b[1],
                        cl.chunks + cl.max_small, b[2]);
  }
  if (threadIdx.x == 0) {
    cl.n_chunks[0] = nskinny + n[1];
    cl.n_chunks[1] = n[2];
    cl.n_chunks[2] = nskinny;
  }
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
    int* __restrict__ counts, int* __restrict__ offsets, ChunkList cl) {
  __shared__ int lds[48];
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
  // the experts' offsets, and (for the chunk list) how many qualify for the small part
  const bool own = q == 0 && mine;
  const int v[2] = {own ? cnt : 0, own ? small_chunks_of(cnt, cl.small_rows) : 0};
  int ex[2], tot[2];
  block_scan<2>(v, ex, tot, lds);
  const int off = ex[0];
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
  if (cl.chunks == nullptr) return;
  build_chunk_list(own, e, off, cnt, cl, tot[1], lds);
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
                          const ChunkList& cl, hipStream_t s) {
  const int S = T * k;
  const int ntiles = (S + kPermTile - 1) / kPermTile;
  permute_count_kernel<<<ntiles, kPermThreads, E * sizeof(int), s>>>(ids, S, E, tile_hist);
  int Ep = 1;
  while (Ep < E) Ep <<= 1;  // E <= 1024
  permute_scan_kernel<<<1, 1024, 0, s>>>(tile_hist, ntiles, E, 1024 / Ep, tile_base, counts,
                                         offsets, cl);
  const size_t scatter_lds = kScatterThreads * sizeof(int) + ((size_t)kScatterWaves * E + 3) / 4 * 4;
  permute_scatter_kernel<<<ntiles, kScatterThreads, scatter_lds, s>>>(ids, S, E, tile_base,
                                                                      sorted_slot, slot_pos);
  return hipGetLastError();
}

// One workgroup of 1024 threads, thread e = expert.
__global__ __launch_bounds__(1024) void chunks_from_offsets_kernel(const int* __restrict__ offsets,
                                                                  int E, ChunkList cl) {
  __shared__ int lds[48];
  const int e = threadIdx.x;
  const bool mine = e < E;
  const int off = mine ? offsets[e] : 0, cnt = mine ? offsets[e + 1] - off : 0;
  const int v[1] = {mine ? small_chunks_of(cnt, cl.small_rows) : 0};
  int ex[1], nsmall[1];
  block_scan<1>(v, ex, nsmall, lds);
  build_chunk_list(mine, e, off, cnt, cl, nsmall[0], lds);
}

hipError_t launch_chunks_from_offsets(const int* offsets, int E, const ChunkList& cl, hipStream_t s) {
  chunks_from_offsets_kernel<<<1, 1024, 0, s>>>(offsets, E, cl);
  return hipGetLastError();
}

}  // namespace strata
