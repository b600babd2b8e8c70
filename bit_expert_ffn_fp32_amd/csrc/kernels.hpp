// Launchers of the gfx950 kernels (host side).  Arguments are validated by the C ABI layer
// before any of these is called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct strata_moe_expert_stats;

namespace strata {

// Chunk of one expert's segment of the sorted slot order, processed by one GEMM work unit.
struct Chunk {
  int32_t expert;
  int32_t row_start;  // first sorted position
  int32_t nrows;      // 1..kChunkRows
  int32_t pad;
};

constexpr int kChunkRows = 224;      // rows of one GEMM work unit (at most 7 fragments of 32)
constexpr int kChunkRowsSmall = 64;  // the same for the small-fragment GEMMs (at most 2)
constexpr int kPermTile = 1024;      // slots per permute tile
constexpr int kSkinnyRows = 32;      // rows of a chunk the skinny GEMMs take (one fragment)
// When at most this many experts of the small part have more than kSkinnyRows rows, each of them
// becomes two skinny chunks (its weights are streamed twice) instead of a small-fragment chunk: a
// small-fragment launch of a few units runs alone after the skinny one (at T = 1024, about 3 such
// experts cost 36 + 23 us), while streaming their weights once more costs well under 1 us each.
constexpr int kSkinnySplitMax = 64;

// The grouped GEMMs' chunk list has two parts.  An expert with at most small_rows rows gets one
// chunk in the small part, run by the small-fragment GEMMs (two workgroups per CU, so that one's
// stage barriers and copy waits overlap the other's matrix work); an expert with more rows gets
// chunks of up to kChunkRows rows (32-row fragments spread evenly) in the large part, whose units
// read the expert's weights once for up to 224 rows.  The two parts run as two launches, so a
// small part of few units would run alone at low occupancy: the list builder uses it only when
// at least min_small experts qualify (enough units to fill the CUs once), else every expert goes
// to the large part.  small_rows is kChunkRowsSmall while the slots average at most 128 rows per
// expert, else 0 (no small part).  Measured at H = 3072, E = 512, k = 10: small chunks for every
// expert beat the large ones up to T = 3072 (60 rows per expert) and lose at T = 4096 (80); with
// skewed routing the large part keeps the hot experts' weights from being re-read per 64 rows.
inline int small_chunk_rows(int64_t S, int64_t E) { return S <= 128 * E ? kChunkRowsSmall : 0; }
// Experts the small part needs: units (one per 128 gate/up outputs) for two workgroups per CU.
inline int min_small_experts(int I) { return (2 * 256 + I / 128 - 1) / (I / 128); }
inline int64_t max_small_chunks(int64_t S, int64_t E, int small_rows) {
  if (!small_rows) return 0;
  const int64_t split = S / (kSkinnyRows + 1) < kSkinnySplitMax ? S / (kSkinnyRows + 1) : kSkinnySplitMax;
  return (E < S ? E : S) + split;  // one chunk per expert, plus the second halves of split ones
}
// Chunks of the small part that run on the small-fragment GEMMs: its experts of more than
// kSkinnyRows rows, and only when more than kSkinnySplitMax of them exist (else they are split for
// the skinny GEMMs).  None when S slots cannot give kSkinnySplitMax + 1 experts kSkinnyRows + 1
// rows each, so those launches are skipped; else at most S / (kSkinnyRows + 1).
inline int64_t max_rest_chunks(int64_t S, int64_t max_small) {
  if (S < (int64_t)(kSkinnySplitMax + 1) * (kSkinnyRows + 1)) return 0;
  const int64_t n = S / (kSkinnyRows + 1);
  return n < max_small ? n : max_small;
}
inline int64_t max_large_chunks(int64_t S, int64_t E, int small_rows, int min_small) {
  // experts in the large part: those with more than small_rows rows, plus (when the small part
  // is not used) fewer than min_small others
  int64_t n = S / (small_rows + 1) + (small_rows ? min_small : 0);
  n = n < E ? n : E;
  return S / kChunkRows + (n < S ? n : S) + 1;
}

// Number of chunks of an expert with cnt rows in the small and in the large part.
__device__ __forceinline__ int small_chunks_of(int cnt, int small_rows) { return cnt > 0 && cnt <= small_rows ? 1 : 0; }
__device__ __forceinline__ int large_chunks_of(int cnt, int small_rows) {
  if (cnt <= small_rows) return 0;
  const int nfrag = (cnt + 31) / 32;
  return (nfrag + kChunkRows / 32 - 1) / (kChunkRows / 32);
}
// Writes the chunks of expert e, whose rows are sorted positions [off, off + cnt): at small[sb]
// or at large[lb ..].
__device__ __forceinline__ void write_expert_chunks(int e, int off, int cnt, int small_rows,
                                                   Chunk* small, int sb, Chunk* large, int lb) {
  if (cnt <= 0) return;
  if (cnt <= small_rows) {
    small[sb] = Chunk{e, off, cnt, 0};
    return;
  }
  const int nfrag = (cnt + 31) / 32, nch = large_chunks_of(cnt, small_rows);
  const int fb = nfrag / nch, extra = nfrag % nch;
  int row = off, used = 0;
  for (int c = 0; c < nch; ++c) {
    const int nf = fb + (c < extra ? 1 : 0);
    const int rows = min(nf * 32, cnt - used * 32);
    large[lb + c] = Chunk{e, row, rows, 0};
    row += rows;
    used += nf;
  }
}

// Row-major -> tiled weight layout for n_mat matrices of R x K (R a multiple of 4, K of 64).
hipError_t launch_pack(int fmt, int n_mat, int R, int K, const void* codes, const uint16_t* scales,
                       void* tcodes, uint16_t* tscales, hipStream_t s);

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t s);

// Where the chunk list goes and how it is split (small_chunk_rows, min_small_experts,
// max_small_chunks): the small part at chunks[0 ..) with its count in n_chunks[0], the large part
// at chunks[max_small ..) with its count in n_chunks[1].  The small part lists its chunks of at
// most kSkinnyRows rows first (their count in n_chunks[2]; an expert split under kSkinnySplitMax
// gives two consecutive ones); those run on the skinny GEMMs, the rest of the small part on the
// small-fragment GEMMs.
struct ChunkList {
  Chunk* chunks;
  int* n_chunks;
  int small_rows;
  int min_small;
  int max_small;
};

// Stable counting sort; also writes the GEMM chunk list when cl.chunks != NULL.
hipError_t launch_permute(const int* ids, int T, int E, int k, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, int* tile_hist, int* tile_base,
                          const ChunkList& cl, hipStream_t s);

// The GEMM chunk list from the offsets [E + 1] of a counting sort (E <= 1024).
hipError_t launch_chunks_from_offsets(const int* offsets, int E, const ChunkList& cl, hipStream_t s);

// Per-token range of the fp16 activations of the grouped GEMM: x16 = x * 2^sx with the row's
// largest |x| in [2^14, 2^15) (sx = 0 for an all-zero row), n2 = sum of x16^2 in fp32.
struct XInfo {
  int32_t sx;
  float n2;
};

// x bf16 [T][H] -> fp16 (scaled per token) in the fragment order of the grouped GEMM (see
// prefill.hip), and each token's XInfo.
hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, XInfo* xinfo,
                           hipStream_t s);
// launch_route and launch_x_to_f16 in one launch (T >= 1).
hipError_t launch_route_x16(const float* logits, int T, int E, int k, int* ids, float* w,
                            const uint16_t* x, int H, uint16_t* x16, XInfo* xinfo, hipStream_t s);

// S: the number of slots (sizes the work units; the chunk list itself is read on the device).
// chunks / n_chunks: the two-part list of launch_permute, with max_small and max_large its parts'
// capacities; the small part runs on the skinny and the small-fragment GEMMs (if max_small > 0),
// then the large.
hipError_t launch_ffn_up(int fmt, const uint16_t* x16, const XInfo* xinfo, const int* sorted_slot,
                         int k, int64_t S, const Chunk* chunks, const int* n_chunks, int max_small,
                         int max_large,
                         const void* gate_codes, const void* up_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, const strata_moe_expert_stats* stats, int E,
                         int H, int I, uint16_t* a16, hipStream_t s);

hipError_t launch_ffn_down(int fmt, const uint16_t* a16, const XInfo* xinfo,
                           const int* sorted_slot, int k, int64_t S, const Chunk* chunks,
                           const int* n_chunks, int max_small, int max_large,
                           const void* down_codes, const uint16_t* down_scales,
                           const strata_moe_expert_stats* stats, int E, int H, int I,
                           uint16_t* expert_out, hipStream_t s);

// Range statistics of a layer's tiled weights, one strata_moe_expert_stats per expert.
hipError_t launch_weight_stats(int fmt, int E, int H, int I, const void* gate_codes,
                               const void* up_codes, const void* down_codes,
                               const uint16_t* gate_scales, const uint16_t* up_scales,
                               const uint16_t* down_scales, strata_moe_expert_stats* stats,
                               hipStream_t s);

hipError_t launch_combine(const uint16_t* expert_out, const float* w, int T, int k, int H,
                          float* y, int accumulate, hipStream_t s);

hipError_t launch_rmsnorm(const float* h, int T, int H, float eps, uint16_t* x, hipStream_t s);

// Dense bf16 layers.  Router: logits fp32 [T][E] = x W_r^T.  Shared expert: a = bf16(SiLU(x W_sg^T)
// * (x W_su^T)) into a [T][I], then y (+)= a W_sd^T.  H and I multiples of 64.
// Router projection and shared-expert gate/up GEMV in one launch (T <= 8 token rows; see
// router_shared_up_fits): logits fp32 [T][E] = x W_r^T, a bf16 [T][Is] = SiLU(x W_sg^T) * (x W_su^T).
bool router_shared_up_fits(int T, int H);
hipError_t launch_router_shared_up(const uint16_t* x, const uint16_t* wr, int E, const uint16_t* wg,
                                   const uint16_t* wu, int Is, int T, int H, float* logits,
                                   uint16_t* a, hipStream_t s);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                                float* logits, hipStream_t s);
hipError_t launch_shared_expert(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                                const uint16_t* wd, int T, int H, int I, float* y, int accumulate,
                                uint16_t* a, hipStream_t s);

// Expert usage: usage[e] += slots of ids routed to e (E <= 1024); order = experts by usage, most
// used first, ties to the lower index.
hipError_t launch_usage_update(const int* ids, int64_t S, int E, uint64_t* usage, hipStream_t s);
hipError_t launch_usage_rank(const uint64_t* usage, int E, int* order, hipStream_t s);

// Decode path (T <= 8).  With h_res != NULL the input is the residual stream h (fp32 [T][H]) and
// x = bf16(h / sqrt(mean(h^2) + eps)) is formed in the first kernel (x is then unused).  With
// a_sh != NULL (and h_res == NULL) the first kernel also applies a shared expert's down projection,
// y (=|+= by accumulate) a_sh W_sd^T (a_sh bf16 [T][Is], W_sd bf16 [H][Is], Is % 8 == 0), and the
// routed output is then added to y.
hipError_t launch_decode(int fmt, const uint16_t* x, const float* h_res, float eps,
                         const float* logits, int T, int E, int k,
                         int H, int I, const void* gate_codes, const void* up_codes,
                         const void* down_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, const uint16_t* down_scales, float* y,
                         int accumulate, int* ids, float* w, void* ws, hipStream_t s,
                         const uint16_t* a_sh = nullptr, const uint16_t* w_sd = nullptr,
                         int Is = 0);
size_t decode_workspace_bytes(int T, int E, int k, int H, int I);
// The decode path's fixed scratch (a device array of the library, one per GPU): its size, and
// the current device's address of it (looked up on first use per device).
size_t decode_static_scratch_bytes();
hipError_t decode_static_scratch(void** ptr);
// Whether the decode kernels take this shape (T <= 8, T*k <= 128, H <= 4096, I <= 4096 and the
// staged activations fit in LDS).
bool decode_fits(int T, int E, int k, int H, int I);

}  // namespace strata
