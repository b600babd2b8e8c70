// C ABI of the MoE expert layer: argument validation, workspace layout and kernel dispatch.
// Every check runs before the first HIP call, so an error return means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "kernels.hpp"
#include "strata_moe.h"

using strata::Chunk;

// The weights struct's layout is part of the ABI (field order as documented in the header).
static_assert(offsetof(strata_moe_weights, fmt) == 0 && offsetof(strata_moe_weights, num_experts) == 4 &&
              offsetof(strata_moe_weights, hidden) == 8 && offsetof(strata_moe_weights, inter) == 12 &&
              offsetof(strata_moe_weights, gate_codes) == 16 && offsetof(strata_moe_weights, up_codes) == 24 &&
              offsetof(strata_moe_weights, gate_scales) == 32 && offsetof(strata_moe_weights, up_scales) == 40 &&
              offsetof(strata_moe_weights, down_codes) == 48 && offsetof(strata_moe_weights, down_scales) == 56 &&
              offsetof(strata_moe_weights, stats) == 64 && sizeof(strata_moe_weights) == 72,
              "strata_moe_weights layout");
static_assert(sizeof(strata_moe_expert_stats) == 16, "strata_moe_expert_stats layout");

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;
constexpr int kMaxDecodeT = 8;
// Up to this many tokens the one-call layer runs the decode path on slices of at most
// kMaxDecodeT tokens: the tokens of a layer are independent, and streaming each touched expert
// once per slice still beats the grouped GEMMs while experts see only a few rows each (at
// H = 3072, E = 512, k = 10, I = 768 the two tie at T = 32 and the GEMMs win from T = 40 on).
constexpr int kSplitDecodeMaxT = 32;

size_t round_up(size_t b) { return (b + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool shape_ok(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return false;
  if ((int64_t)T * k > INT32_MAX / 2) return false;
  return true;
}

strata_status check_route_shape(int32_t T, int32_t E, int32_t k) {
  if (!shape_ok(T, E, k) || k > E) return STRATA_ERR_INVALID_ARGUMENT;
  if (E > kMaxE || k > kMaxK) return STRATA_ERR_UNSUPPORTED;
  return STRATA_OK;
}

strata_status check_weights(const strata_moe_weights* w) {
  if (!w) return STRATA_ERR_INVALID_ARGUMENT;
  if (w->fmt != STRATA_Q2_B32 && w->fmt != STRATA_Q3_B32) return STRATA_ERR_INVALID_ARGUMENT;
  if (w->num_experts < 1 || w->hidden < 1 || w->inter < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if (w->hidden % 32 || w->inter % 32) return STRATA_ERR_INVALID_ARGUMENT;
  if (w->num_experts > kMaxE) return STRATA_ERR_UNSUPPORTED;
  if (w->hidden % 256 || w->inter % 128) return STRATA_ERR_UNSUPPORTED;
  const void* ptrs[6] = {w->gate_codes, w->up_codes, w->down_codes,
                         w->gate_scales, w->up_scales, w->down_scales};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  return STRATA_OK;
}

// The prefill path also needs the weights' range statistics.
strata_status check_stats(const strata_moe_weights* w) {
  return w->stats && aligned16(w->stats) ? STRATA_OK : STRATA_ERR_INVALID_ARGUMENT;
}

strata_status from_hip(hipError_t e) { return e == hipSuccess ? STRATA_OK : STRATA_ERR_HIP; }

// Workspace of the prefill path, carved in this order (each piece 256-byte aligned).
struct PrefillWs {
  int* ids;
  float* w;
  int* counts;
  int* offsets;
  int* sorted_slot;
  int* slot_pos;
  int* tile_hist;
  int* tile_base;
  Chunk* chunks;
  int* n_chunks;
  strata::XInfo* xinfo;
  uint16_t* x16;
  uint16_t* a16;
  uint16_t* expert_out;
  size_t bytes;
  strata::ChunkList cl;  // the chunk list's parts: chunks, n_chunks, small_rows, min_small, max_small
  int max_large;
};

PrefillWs carve_prefill(void* base, int32_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  PrefillWs p{};
  const size_t S = (size_t)T * k;
  const size_t ntiles = (S + strata::kPermTile - 1) / strata::kPermTile;
  p.cl.small_rows = strata::small_chunk_rows((int64_t)S, E);
  p.cl.min_small = strata::min_small_experts(I);
  p.cl.max_small = (int)strata::max_small_chunks((int64_t)S, E, p.cl.small_rows);
  p.max_large = (int)strata::max_large_chunks((int64_t)S, E, p.cl.small_rows, p.cl.min_small);
  uint8_t* c = static_cast<uint8_t*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = c ? c + off : nullptr;
    off += round_up(bytes);
    return r;
  };
  p.ids = static_cast<int*>(take(S * 4));
  p.w = static_cast<float*>(take(S * 4));
  p.counts = static_cast<int*>(take((size_t)E * 4));
  p.offsets = static_cast<int*>(take((size_t)(E + 1) * 4));
  p.sorted_slot = static_cast<int*>(take(S * 4));
  p.slot_pos = static_cast<int*>(take(S * 4));
  p.tile_hist = static_cast<int*>(take(ntiles * E * 4));
  p.tile_base = static_cast<int*>(take(ntiles * E * 4));
  p.chunks = static_cast<Chunk*>(take((size_t)(p.cl.max_small + p.max_large) * sizeof(Chunk)));
  p.n_chunks = static_cast<int*>(take(16));
  p.cl.chunks = p.chunks;
  p.cl.n_chunks = p.n_chunks;
  p.xinfo = static_cast<strata::XInfo*>(take((size_t)T * sizeof(strata::XInfo)));
  p.x16 = static_cast<uint16_t*>(take((size_t)T * H * 2));
  p.a16 = static_cast<uint16_t*>(take(S * I * 2));
  p.expert_out = static_cast<uint16_t*>(take(S * H * 2));
  p.bytes = off;
  return p;
}


// Decode paths (T <= kSplitDecodeMaxT): the decode kernels' workspace for slices of at most
// kMaxDecodeT tokens, then, for a caller that asks strata_moe_layer for the permutation, the
// routing result of all T tokens and one counting sort's outputs and scratch.
struct DecodePermWs {
  int* ids;
  int* counts;
  int* offsets;
  int* sorted_slot;
  int* slot_pos;
  int* tile_hist;
  int* tile_base;
  size_t bytes;
};

DecodePermWs carve_decode_perm(void* base, int32_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  DecodePermWs q{};
  const size_t S = (size_t)T * k;
  const size_t ntiles = (S + strata::kPermTile - 1) / strata::kPermTile;
  const int32_t td = T < kMaxDecodeT ? T : kMaxDecodeT;
  uint8_t* c = static_cast<uint8_t*>(base);
  size_t off = round_up(strata::decode_workspace_bytes(td, E, k, H, I));
  auto take = [&](size_t bytes) {
    void* r = c ? c + off : nullptr;
    off += round_up(bytes);
    return r;
  };
  q.ids = static_cast<int*>(take(S * 4));
  q.counts = static_cast<int*>(take((size_t)E * 4));
  q.offsets = static_cast<int*>(take((size_t)(E + 1) * 4));
  q.sorted_slot = static_cast<int*>(take(S * 4));
  q.slot_pos = static_cast<int*>(take(S * 4));
  q.tile_hist = static_cast<int*>(take(ntiles * E * 4));
  q.tile_base = static_cast<int*>(take(ntiles * E * 4));
  q.bytes = off;
  return q;
}

}  // namespace

extern "C" {

const char* strata_status_string(strata_status st) {
  switch (st) {
    case STRATA_OK: return "ok";
    case STRATA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case STRATA_ERR_UNSUPPORTED: return "unsupported shape";
    case STRATA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case STRATA_ERR_HIP: return "HIP launch error";
    default: break;
  }
  return "unknown status";
}

// The size queries answer 0 for every (T, E, k) the compute calls reject, which also keeps the
// sizes' intermediate counts (E + 1 offsets, the chunk bounds) inside int.
size_t strata_moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t k) {
  if (check_route_shape(T, E, k) != STRATA_OK) return 0;
  const size_t S = (size_t)T * k;
  const size_t ntiles = (S + strata::kPermTile - 1) / strata::kPermTile;
  return 2 * round_up(ntiles * E * 4);
}

size_t strata_moe_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  if (check_route_shape(T, E, k) != STRATA_OK || H < 1 || I < 1) return 0;
  const size_t pre = carve_prefill(nullptr, T, E, k, H, I).bytes;
  const size_t dec = T <= kSplitDecodeMaxT ? carve_decode_perm(nullptr, T, E, k, H, I).bytes : 0;
  return pre > dec ? pre : dec;
}

strata_status strata_moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                               int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  strata_status st = check_route_shape(T, E, k);
  if (st != STRATA_OK) return st;
  if (T == 0) return STRATA_OK;
  if (!logits || !topk_ids || !topk_w) return STRATA_ERR_INVALID_ARGUMENT;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_route(logits, T, E, k, topk_ids, topk_w, stream));
}

strata_status strata_moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                 int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  strata_status st = check_route_shape(T, E, k);
  if (st != STRATA_OK) return st;
  if (T == 0) return STRATA_OK;
  const void* ptrs[6] = {topk_ids, counts, offsets, sorted_slot, slot_pos, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  const size_t need = strata_moe_permute_workspace_bytes(T, E, k);
  if (workspace_bytes < need) return STRATA_ERR_WORKSPACE_TOO_SMALL;
  const size_t S = (size_t)T * k;
  const size_t ntiles = (S + strata::kPermTile - 1) / strata::kPermTile;
  int* hist = static_cast<int*>(workspace);
  int* base = reinterpret_cast<int*>(static_cast<uint8_t*>(workspace) + round_up(ntiles * E * 4));
  return from_hip(strata::launch_permute(topk_ids, T, E, k, counts, offsets, sorted_slot, slot_pos,
                                         hist, base, strata::ChunkList{}, stream));
}

strata_status strata_moe_expert_ffn(const strata_moe_weights* w, const uint16_t* x, int32_t T,
                                    int32_t k, const int32_t* offsets, const int32_t* sorted_slot,
                                    uint16_t* expert_out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  st = check_route_shape(T, w->num_experts, k);
  if (st != STRATA_OK) return st;
  if (T == 0) return STRATA_OK;
  const void* ptrs[5] = {x, offsets, sorted_slot, expert_out, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  st = check_stats(w);
  if (st != STRATA_OK) return st;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (workspace_bytes < strata_moe_workspace_bytes(T, E, k, H, I)) return STRATA_ERR_WORKSPACE_TOO_SMALL;
  PrefillWs p = carve_prefill(workspace, T, E, k, H, I);
  hipError_t e = strata::launch_chunks_from_offsets(offsets, E, p.cl, stream);
  if (e == hipSuccess) e = strata::launch_x_to_f16(x, T, H, p.x16, p.xinfo, stream);
  if (e == hipSuccess)
    e = strata::launch_ffn_up(w->fmt, p.x16, p.xinfo, sorted_slot, k, (int64_t)T * k, p.chunks,
                              p.n_chunks, p.cl.max_small, p.max_large, w->gate_codes, w->up_codes,
                              w->gate_scales, w->up_scales, w->stats, E, H, I, p.a16, stream);
  if (e == hipSuccess)
    e = strata::launch_ffn_down(w->fmt, p.a16, p.xinfo, sorted_slot, k, (int64_t)T * k, p.chunks,
                                p.n_chunks, p.cl.max_small, p.max_large, w->down_codes, w->down_scales, w->stats,
                                E, H, I, expert_out, stream);
  return from_hip(e);
}

strata_status strata_moe_combine(const uint16_t* expert_out, const float* topk_w, int32_t T,
                                 int32_t k, int32_t H, float* y, int32_t accumulate,
                                 hipStream_t stream) {
  if (T < 0 || k < 1 || H < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if ((int64_t)T * k > INT32_MAX / 2) return STRATA_ERR_INVALID_ARGUMENT;
  if (H % 8) return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  if (!expert_out || !topk_w || !y) return STRATA_ERR_INVALID_ARGUMENT;
  if (!aligned16(expert_out) || !aligned16(topk_w) || !aligned16(y)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_combine(expert_out, topk_w, T, k, H, y, accumulate, stream));
}

strata_status strata_moe_decode(const strata_moe_weights* w, const uint16_t* x, const float* logits,
                                int32_t T, int32_t k, float* y, int32_t accumulate,
                                int32_t* opt_topk_ids, float* opt_topk_w, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  st = check_route_shape(T, w->num_experts, k);
  if (st != STRATA_OK) return st;
  if (T > kMaxDecodeT) return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  if (!strata::decode_fits(T, w->num_experts, k, w->hidden, w->inter)) return STRATA_ERR_UNSUPPORTED;
  const void* ptrs[4] = {x, logits, y, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  if ((opt_topk_ids && !aligned16(opt_topk_ids)) || (opt_topk_w && !aligned16(opt_topk_w)))
    return STRATA_ERR_INVALID_ARGUMENT;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (workspace_bytes < strata_moe_workspace_bytes(T, E, k, H, I)) return STRATA_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(strata::launch_decode(w->fmt, x, nullptr, 0.0f, logits, T, E, k, H, I,
                                        w->gate_codes, w->up_codes,
                                        w->down_codes, w->gate_scales, w->up_scales, w->down_scales,
                                        y, accumulate, opt_topk_ids, opt_topk_w, workspace, stream));
}

strata_status strata_moe_decode_static(const strata_moe_weights* w, const uint16_t* x,
                                       const float* logits, int32_t T, int32_t k, float* y,
                                       int32_t accumulate, int32_t* opt_topk_ids,
                                       float* opt_topk_w, hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  st = check_route_shape(T, w->num_experts, k);
  if (st != STRATA_OK) return st;
  if (T > kMaxDecodeT) return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (!strata::decode_fits(T, E, k, H, I)) return STRATA_ERR_UNSUPPORTED;
  const void* ptrs[3] = {x, logits, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  if ((opt_topk_ids && !aligned16(opt_topk_ids)) || (opt_topk_w && !aligned16(opt_topk_w)))
    return STRATA_ERR_INVALID_ARGUMENT;
  if (strata::decode_workspace_bytes(T, E, k, H, I) > strata::decode_static_scratch_bytes())
    return STRATA_ERR_WORKSPACE_TOO_SMALL;
  void* scratch = nullptr;
  if (strata::decode_static_scratch(&scratch) != hipSuccess) return STRATA_ERR_HIP;
  return from_hip(strata::launch_decode(w->fmt, x, nullptr, 0.0f, logits, T, E, k, H, I,
                                        w->gate_codes, w->up_codes, w->down_codes, w->gate_scales,
                                        w->up_scales, w->down_scales, y, accumulate, opt_topk_ids,
                                        opt_topk_w, scratch, stream));
}

size_t strata_moe_decode_static_max_bytes(void) { return strata::decode_static_scratch_bytes(); }

strata_status strata_moe_layer(const strata_moe_weights* w, const uint16_t* x, const float* logits,
                               int32_t T, int32_t k, float* y, int32_t accumulate,
                               int32_t* opt_topk_ids, float* opt_topk_w, int32_t* opt_counts,
                               int32_t* opt_offsets, int32_t* opt_sorted_slot, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  st = check_route_shape(T, w->num_experts, k);
  if (st != STRATA_OK) return st;
  if (T == 0) return STRATA_OK;
  const void* ptrs[4] = {x, logits, y, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  const void* opts[5] = {opt_topk_ids, opt_topk_w, opt_counts, opt_offsets, opt_sorted_slot};
  for (const void* p : opts)
    if (p && !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (workspace_bytes < strata_moe_workspace_bytes(T, E, k, H, I)) return STRATA_ERR_WORKSPACE_TOO_SMALL;
  const bool want_perm = opt_counts || opt_offsets || opt_sorted_slot;
  const bool decode_path =
      (T <= kMaxDecodeT && strata::decode_fits(T, E, k, H, I)) ||
      (T <= kSplitDecodeMaxT && strata::decode_fits(kMaxDecodeT, E, k, H, I));
  if (decode_path) {
    // Balanced slices of at most kMaxDecodeT tokens in token order on the same stream (the
    // slices share the workspace one after the other).  The decode kernels read x with 16-byte
    // loads (a slice starts at a multiple of H >= 256 values) and logits, ids and weights per
    // element.
    const DecodePermWs q = carve_decode_perm(workspace, T, E, k, H, I);
    int* ids = opt_topk_ids ? opt_topk_ids : (want_perm ? q.ids : nullptr);
    const int32_t n = (T + kMaxDecodeT - 1) / kMaxDecodeT;
    int32_t t0 = 0;
    hipError_t e = hipSuccess;
    for (int32_t i = 0; i < n && e == hipSuccess; ++i) {
      const int32_t ts = T / n + (i < T % n ? 1 : 0);
      e = strata::launch_decode(w->fmt, x + (size_t)t0 * H, nullptr, 0.0f, logits + (size_t)t0 * E, ts,
                                E, k, H, I, w->gate_codes, w->up_codes, w->down_codes,
                                w->gate_scales, w->up_scales, w->down_scales, y + (size_t)t0 * H,
                                accumulate, ids ? ids + (size_t)t0 * k : nullptr,
                                opt_topk_w ? opt_topk_w + (size_t)t0 * k : nullptr, workspace,
                                stream);
      t0 += ts;
    }
    if (e == hipSuccess && want_perm)
      e = strata::launch_permute(ids, T, E, k, opt_counts ? opt_counts : q.counts,
                                 opt_offsets ? opt_offsets : q.offsets,
                                 opt_sorted_slot ? opt_sorted_slot : q.sorted_slot, q.slot_pos,
                                 q.tile_hist, q.tile_base, strata::ChunkList{}, stream);
    return from_hip(e);
  }
  st = check_stats(w);
  if (st != STRATA_OK) return st;
  PrefillWs p = carve_prefill(workspace, T, E, k, H, I);
  int* ids = opt_topk_ids ? opt_topk_ids : p.ids;
  float* rw = opt_topk_w ? opt_topk_w : p.w;
  int* counts = opt_counts ? opt_counts : p.counts;
  int* offsets = opt_offsets ? opt_offsets : p.offsets;
  int* sorted = opt_sorted_slot ? opt_sorted_slot : p.sorted_slot;
  hipError_t e = strata::launch_route_x16(logits, T, E, k, ids, rw, x, H, p.x16, p.xinfo, stream);
  if (e == hipSuccess)
    e = strata::launch_permute(ids, T, E, k, counts, offsets, sorted, p.slot_pos, p.tile_hist,
                               p.tile_base, p.cl, stream);
  if (e == hipSuccess)
    e = strata::launch_ffn_up(w->fmt, p.x16, p.xinfo, sorted, k, (int64_t)T * k, p.chunks,
                              p.n_chunks, p.cl.max_small, p.max_large, w->gate_codes, w->up_codes,
                              w->gate_scales, w->up_scales, w->stats, E, H, I, p.a16, stream);
  if (e == hipSuccess)
    e = strata::launch_ffn_down(w->fmt, p.a16, p.xinfo, sorted, k, (int64_t)T * k, p.chunks,
                                p.n_chunks, p.cl.max_small, p.max_large, w->down_codes, w->down_scales, w->stats,
                                E, H, I, p.expert_out, stream);
  if (e == hipSuccess) e = strata::launch_combine(p.expert_out, rw, T, k, H, y, accumulate, stream);
  return from_hip(e);
}

size_t strata_moe_residual_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  const size_t layer = strata_moe_workspace_bytes(T, E, k, H, I);
  if (layer == 0) return 0;
  return round_up(layer) + round_up((size_t)T * H * 2);
}

strata_status strata_moe_layer_residual(const strata_moe_weights* w, float* h, const float* logits,
                                        int32_t T, int32_t k, float eps, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  st = check_route_shape(T, w->num_experts, k);
  if (st != STRATA_OK) return st;
  if (!(eps >= 0.0f)) return STRATA_ERR_INVALID_ARGUMENT;
  if (T == 0) return STRATA_OK;
  const void* ptrs[3] = {h, logits, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (workspace_bytes < strata_moe_residual_workspace_bytes(T, E, k, H, I))
    return STRATA_ERR_WORKSPACE_TOO_SMALL;
  if (T <= kMaxDecodeT && strata::decode_fits(T, E, k, H, I))  // RMSNorm inside the first kernel
    return from_hip(strata::launch_decode(w->fmt, nullptr, h, eps, logits, T, E, k, H, I,
                                          w->gate_codes, w->up_codes, w->down_codes,
                                          w->gate_scales, w->up_scales, w->down_scales, h, 1,
                                          nullptr, nullptr, workspace, stream));
  const size_t layer = round_up(strata_moe_workspace_bytes(T, E, k, H, I));
  uint16_t* x = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + layer);
  hipError_t e = strata::launch_rmsnorm(h, T, H, eps, x, stream);
  if (e != hipSuccess) return STRATA_ERR_HIP;
  return strata_moe_layer(w, x, logits, T, k, h, 1, nullptr, nullptr, nullptr, nullptr, nullptr,
                          workspace, layer, stream);
}

strata_status strata_moe_weight_stats(const strata_moe_weights* w, strata_moe_expert_stats* stats,
                                      hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  if (!stats || !aligned16(stats)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_weight_stats(w->fmt, w->num_experts, w->hidden, w->inter,
                                              w->gate_codes, w->up_codes, w->down_codes,
                                              w->gate_scales, w->up_scales, w->down_scales, stats,
                                              stream));
}

strata_status strata_moe_pack_matrix(int32_t fmt, int32_t n_mat, int32_t rows, int32_t K,
                                    const void* codes, const uint16_t* scales, void* tiled_codes,
                                    uint16_t* tiled_scales, hipStream_t stream) {
  if (fmt != STRATA_Q2_B32 && fmt != STRATA_Q3_B32) return STRATA_ERR_INVALID_ARGUMENT;
  if (n_mat < 1 || rows < 1 || K < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if (rows % 4 || K % 64) return STRATA_ERR_UNSUPPORTED;
  if ((int64_t)n_mat * rows * (K / 64) > (int64_t)INT32_MAX * 64) return STRATA_ERR_UNSUPPORTED;
  const void* ptrs[4] = {codes, scales, tiled_codes, tiled_scales};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  const size_t cb = fmt == STRATA_Q2_B32 ? 8 : 12;
  const size_t nblk = (size_t)n_mat * rows * (K / 32);
  const uintptr_t c0 = (uintptr_t)codes, c1 = c0 + nblk * cb, t0 = (uintptr_t)tiled_codes,
                  t1 = t0 + nblk * cb;
  const uintptr_t s0 = (uintptr_t)scales, s1 = s0 + nblk * 2, u0 = (uintptr_t)tiled_scales,
                  u1 = u0 + nblk * 2;
  if ((c0 < t1 && t0 < c1) || (s0 < u1 && u0 < s1) || (c0 < u1 && u0 < c1) || (s0 < t1 && t0 < s1))
    return STRATA_ERR_INVALID_ARGUMENT;  // overlapping source and destination
  return from_hip(strata::launch_pack(fmt, n_mat, rows, K, codes, scales, tiled_codes,
                                      tiled_scales, stream));
}

size_t strata_moe_shared_workspace_bytes(int32_t T, int32_t I) {
  if (T < 0 || I < 1) return 0;
  return round_up((size_t)T * I * 2);
}

strata_status strata_moe_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t T,
                                       int32_t H, int32_t E, float* logits, hipStream_t stream) {
  if (T < 0 || H < 1 || E < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if (H % 64) return STRATA_ERR_UNSUPPORTED;
  if ((int64_t)T * H > INT32_MAX || (int64_t)E * H > INT32_MAX || (int64_t)T * E > INT32_MAX)
    return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  const void* ptrs[3] = {x, w_router, logits};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_router_logits(x, w_router, T, H, E, logits, stream));
}

strata_status strata_moe_shared_expert(const uint16_t* x, const uint16_t* w_gate,
                                       const uint16_t* w_up, const uint16_t* w_down, int32_t T,
                                       int32_t H, int32_t I, float* y, int32_t accumulate,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (T < 0 || H < 1 || I < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if (H % 64 || I % 64) return STRATA_ERR_UNSUPPORTED;
  if ((int64_t)T * H > INT32_MAX || (int64_t)T * I > INT32_MAX || (int64_t)H * I > INT32_MAX)
    return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  const void* ptrs[6] = {x, w_gate, w_up, w_down, y, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < strata_moe_shared_workspace_bytes(T, I)) return STRATA_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(strata::launch_shared_expert(x, w_gate, w_up, w_down, T, H, I, y, accumulate,
                                               static_cast<uint16_t*>(workspace), stream));
}

size_t strata_moe_block_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                        int32_t Is) {
  const size_t layer = strata_moe_workspace_bytes(T, E, k, H, I);
  if (layer == 0 || Is < 1) return 0;
  return round_up((size_t)T * Is * 2) + round_up(layer);
}

strata_status strata_moe_block(const strata_moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                               const uint16_t* w_router, const uint16_t* w_sgate,
                               const uint16_t* w_sup, const uint16_t* w_sdown, int32_t Is,
                               float* logits, float* y, int32_t accumulate, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  strata_status st = check_weights(w);
  if (st != STRATA_OK) return st;
  st = check_route_shape(T, w->num_experts, k);
  if (st != STRATA_OK) return st;
  if (Is < 1) return STRATA_ERR_INVALID_ARGUMENT;
  const int32_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (Is % 64) return STRATA_ERR_UNSUPPORTED;
  if ((int64_t)T * Is > INT32_MAX || (int64_t)H * Is > INT32_MAX || (int64_t)T * H > INT32_MAX ||
      (int64_t)T * E > INT32_MAX)
    return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  const void* ptrs[8] = {x, w_router, w_sgate, w_sup, w_sdown, logits, y, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return STRATA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < strata_moe_block_workspace_bytes(T, E, k, H, I, Is))
    return STRATA_ERR_WORKSPACE_TOO_SMALL;
  uint16_t* a = static_cast<uint16_t*>(workspace);
  const size_t a_bytes = round_up((size_t)T * Is * 2);
  void* lws = static_cast<uint8_t*>(workspace) + a_bytes;
  const size_t lwb = workspace_bytes - a_bytes;
  if (T <= kMaxDecodeT && strata::decode_fits(T, E, k, H, I) && strata::router_shared_up_fits(T, H)) {
    hipError_t e = strata::launch_router_shared_up(x, w_router, E, w_sgate, w_sup, Is, T, H, logits,
                                                   a, stream);
    if (e != hipSuccess) return STRATA_ERR_HIP;
    return from_hip(strata::launch_decode(w->fmt, x, nullptr, 0.0f, logits, T, E, k, H, I,
                                          w->gate_codes, w->up_codes, w->down_codes,
                                          w->gate_scales, w->up_scales, w->down_scales, y,
                                          accumulate, nullptr, nullptr, lws, stream, a, w_sdown, Is));
  }
  st = strata_moe_router_logits(x, w_router, T, H, E, logits, stream);
  if (st != STRATA_OK) return st;
  st = strata_moe_shared_expert(x, w_sgate, w_sup, w_sdown, T, H, Is, y, accumulate, a, a_bytes,
                                stream);
  if (st != STRATA_OK) return st;
  return strata_moe_layer(w, x, logits, T, k, y, 1, nullptr, nullptr, nullptr, nullptr, nullptr,
                          lws, lwb, stream);
}

strata_status strata_moe_usage_update(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                     uint64_t* usage, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if ((int64_t)T * k > INT32_MAX / 2) return STRATA_ERR_INVALID_ARGUMENT;
  if (E > kMaxE) return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  if (!topk_ids || !usage || !aligned16(topk_ids) || !aligned16(usage)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_usage_update(topk_ids, (int64_t)T * k, E, usage, stream));
}

strata_status strata_moe_usage_rank(const uint64_t* usage, int32_t E, int32_t* order,
                                   hipStream_t stream) {
  if (E < 1) return STRATA_ERR_INVALID_ARGUMENT;
  if (E > kMaxE) return STRATA_ERR_UNSUPPORTED;
  if (!usage || !order || !aligned16(usage) || !aligned16(order)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_usage_rank(usage, E, order, stream));
}

strata_status strata_moe_rmsnorm(const float* h, int32_t T, int32_t H, float eps, uint16_t* x,
                                 hipStream_t stream) {
  if (T < 0 || H < 1 || !(eps >= 0.0f)) return STRATA_ERR_INVALID_ARGUMENT;
  if (H % 4) return STRATA_ERR_UNSUPPORTED;
  if (T == 0) return STRATA_OK;
  if (!h || !x || !aligned16(h) || !aligned16(x)) return STRATA_ERR_INVALID_ARGUMENT;
  return from_hip(strata::launch_rmsnorm(h, T, H, eps, x, stream));
}

}  // extern "C"
