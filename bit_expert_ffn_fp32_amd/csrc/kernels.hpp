// Launchers of the gfx950 kernels (host side).  Arguments are validated by the C ABI layer
// before any of these is called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace strata {

// Chunk of one expert's segment of the sorted slot order, processed by one GEMM work unit.
struct Chunk {
  int32_t expert;
  int32_t row_start;  // first sorted position
  int32_t nrows;      // 1..kChunkRows
  int32_t pad;
};

constexpr int kChunkRows = 224;  // rows of one GEMM work unit (at most 7 fragments of 32)
constexpr int kPermTile = 1024;  // slots per permute tile

// Upper bound of the number of chunks for S slots over E experts.
inline int64_t max_chunks(int64_t S, int64_t E) {
  return S / kChunkRows + (E < S ? E : S) + 1;
}

// Row-major -> tiled weight layout for n_mat matrices of R x K (R a multiple of 4, K of 64).
hipError_t launch_pack(int fmt, int n_mat, int R, int K, const void* codes, const uint16_t* scales,
                       void* tcodes, uint16_t* tscales, hipStream_t s);

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t s);

// Stable counting sort; also writes the GEMM chunk list (chunks, *n_chunks) when chunks != NULL.
hipError_t launch_permute(const int* ids, int T, int E, int k, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, int* tile_hist, int* tile_base,
                          Chunk* chunks, int* n_chunks, hipStream_t s);

// x bf16 [T][H] -> fp16 in the fragment order of the grouped GEMM (see prefill.hip).
hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, hipStream_t s);

// S: the number of slots (sizes the work units; the chunk list itself is read on the device).
hipError_t launch_ffn_up(int fmt, const uint16_t* x16, const int* sorted_slot, int k, int64_t S,
                         const Chunk* chunks, const int* n_chunks, int max_chunks,
                         const void* gate_codes, const void* up_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, int E, int H, int I, uint16_t* a16,
                         hipStream_t s);

hipError_t launch_ffn_down(int fmt, const uint16_t* a16, const int* sorted_slot, int64_t S,
                           const Chunk* chunks, const int* n_chunks, int max_chunks,
                           const void* down_codes, const uint16_t* down_scales, int E, int H,
                           int I, uint16_t* expert_out, hipStream_t s);

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
// Whether the decode kernels take this shape (T <= 8, T*k <= 128, H <= 4096, I <= 4096 and the
// staged activations fit in LDS).
bool decode_fits(int T, int E, int k, int H, int I);

}  // namespace strata
