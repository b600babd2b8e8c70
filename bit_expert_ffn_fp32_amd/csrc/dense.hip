// Dense bf16 layers beside the routed experts: the router projection and the shared expert.
//
// The pages keep a layer's routers and its shared experts on the GPU next to the expert caches
// ("Strata - the details", How it works / memory tiers; "Strata vs Llama.cpp vs vLLM", transcript
// at 09:28).  Both are dense products out = x W^T with x bf16 [M][K] and W bf16 [N][K], both
// K-contiguous:
//  * router: logits fp32 [T][E] = x W_r^T;
//  * shared expert: a = SiLU(x W_sg^T) * (x W_su^T) rounded to bf16 [T][I], then
//    y (+)= a W_sd^T in fp32 [T][H].
//
// Two kernels per product, chosen by the number of token rows M:
//  * M <= 8 (decode / draft verification): a bandwidth-bound GEMV.  A workgroup streams 8 weight
//    rows with 32 lanes per row (16-byte loads, 512 contiguous bytes per row and instruction),
//    keeps the M token rows in LDS and reduces each row's dot products across its 32 lanes.
//  * larger M: an MFMA GEMM, v_mfma_f32_32x32x16_bf16 with fp32 accumulation, tiles of
//    BM = 128 or 256 rows by 128 columns, 64 reduction indices per stage copied global -> LDS
//    with global_load_lds into a ring of stages, one barrier per stage.
//
// The SwiGLU epilogue needs a token's gate and up sums of the same output in one lane: the GEMM's
// 128 weight rows of a tile are [gate o..o+31, up o..o+31, gate o+32..o+63, up o+32..o+63], so a
// wave's two 32-column fragments hold the gate and up projections of the same 32 outputs.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace strata {
namespace {

// ---------------------------------------------------------------------------------------------
// Epilogues.
enum DenseEpi { kEpiStore = 0, kEpiAccum = 1, kEpiSwiglu = 2 };

STRATA_DEVICE float silu_mul_f(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------------------------------------
// MFMA GEMM.

constexpr int kDK = 64;       // reduction indices per stage (128 bytes of a row)
constexpr int kDBN = 128;     // weight rows (output columns) per tile
constexpr int kDLds = 160 * 1024;

template <int WM>
struct DenseCfg {
  static constexpr int kWaves = 2 * WM;                 // WM wave rows x 2 wave columns
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBM = 64 * WM;                   // token rows per tile
  static constexpr int kABytes = kBM * 128;
  static constexpr int kStage = kABytes + kDBN * 128;
  static constexpr int kCopies = (kBM + kDBN) / 8;      // 1 KB copies (8 rows) per stage
  static constexpr int kPer = kCopies / kWaves;         // per wave
  static constexpr int kNBuf = kDLds / kStage < 4 ? kDLds / kStage : 4;
  static constexpr int kPD = kNBuf - 1;                 // stages in flight ahead of the computed one
  static_assert(kCopies % kWaves == 0, "copies per wave");
  static_assert(kNBuf >= 2 && (kPD - 1) * kPer <= 63, "ring");
  static_assert(kBM * 136 * 4 <= kNBuf * kStage, "fp32 output tile staged in the ring");
  static_assert(kBM * 32 % kThreads == 0 && kBM * 8 % kThreads == 0, "epilogue chunks");
};

template <int N>
STRATA_DEVICE void dense_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Waits until at most min(p, PMAX) later stages' copies (PER each) are outstanding.
template <int PER, int PMAX>
STRATA_DEVICE void dense_wait_pending(int p) {
  if constexpr (PMAX <= 0) {
    dense_wait_vmcnt<0>();
  } else {
    if (p >= PMAX) dense_wait_vmcnt<PMAX * PER>();
    else dense_wait_pending<PER, PMAX - 1>(p);
  }
}

// LDS tile layout: row r (128 bytes = 8 pieces of 8 bf16) keeps piece c in slot c ^ ((r >> 1) & 7),
// so the 16 lanes that one LDS cycle serves (16 consecutive rows, one piece each) hit 64 distinct
// banks.  A 1 KB copy instruction fills 8 rows; lane i lands in row i / 8, slot i % 8.
STRATA_DEVICE int dense_piece(int row, int slot) { return slot ^ ((row >> 1) & 7); }

struct DenseArgs {
  const uint16_t* a;     // [M][K]
  const uint16_t* b0;    // [N][K] (SwiGLU: gate [I][K])
  const uint16_t* b1;    // SwiGLU: up [I][K]; otherwise unused
  void* out;
  int M, N, K;           // N: output columns (SwiGLU: I)
  int accumulate;
};

// Copies stage ks (this wave's kPer pieces of 1 KB) into its ring buffer.
template <int WM>
STRATA_DEVICE void dense_issue(uint8_t* lds, const uint16_t* const* src, int ks) {
  using C = DenseCfg<WM>;
  const int wave = threadIdx.x >> 6;
  uint8_t* st = lds + (ks % C::kNBuf) * C::kStage;
#pragma unroll
  for (int i = 0; i < C::kPer; ++i) {
    const int q = wave + C::kWaves * i;
    __builtin_amdgcn_global_load_lds(src[i] + (size_t)ks * kDK, st + q * 1024, 16, 0, 0);
  }
}

template <int WM, int EPI>
__global__ __launch_bounds__(DenseCfg<WM>::kThreads) void dense_gemm_kernel(DenseArgs p) {
  using C = DenseCfg<WM>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nN = EPI == kEpiSwiglu ? (p.N + 63) / 64 : (p.N + kDBN - 1) / kDBN;
  const int nM = (p.M + C::kBM - 1) / C::kBM;
  const int nT = nM * nN;
  // consecutive tiles (same token rows, neighbouring columns) go to the same XCD
  int t = blockIdx.x;
  if ((nT & 7) == 0) t = (t & 7) * (nT >> 3) + (t >> 3);
  const int tm = t / nN, tn = t - tm * nN;
  const int m0 = tm * C::kBM;

  // this lane's source row of each of its copies
  const uint16_t* src[C::kPer];
#pragma unroll
  for (int i = 0; i < C::kPer; ++i) {
    const int q = wave + C::kWaves * i;            // copy index: A rows first, then weight rows
    const int r = 8 * q + (lane >> 3);             // tile row (A rows 0..BM-1, then B rows)
    const int piece = dense_piece(r, lane & 7);
    const uint16_t* row;
    if (r < C::kBM) {
      const int m = min(m0 + r, p.M - 1);
      row = p.a + (size_t)m * p.K;
    } else {
      const int rb = r - C::kBM;
      if constexpr (EPI == kEpiSwiglu) {
        const int o = min(tn * 64 + (rb >> 6) * 32 + (rb & 31), p.N - 1);
        row = ((rb >> 5) & 1 ? p.b1 : p.b0) + (size_t)o * p.K;
      } else {
        const int n = min(tn * kDBN + rb, p.N - 1);
        row = p.b0 + (size_t)n * p.K;
      }
    }
    src[i] = row + piece * 8;
  }

  const int nk = p.K / kDK;
#pragma unroll
  for (int s = 0; s < C::kPD; ++s)
    if (s < nk) dense_issue<WM>(lds, src, s);

  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 31, hh = lane >> 5;
  const int key = (m >> 1) & 7;
  f32x16_t acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.0f;

  for (int ks = 0; ks < nk; ++ks) {
    dense_wait_pending<C::kPer, C::kPD - 1>(nk - 1 - ks);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read of this stage moves above the barrier
    if (ks + C::kPD < nk) dense_issue<WM>(lds, src, ks + C::kPD);
    const uint8_t* st = lds + (ks % C::kNBuf) * C::kStage;
    const uint8_t* at = st + (wm * 64 + m) * 128;
    const uint8_t* bt = st + C::kABytes + (wn * 64 + m) * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int slot = ((hh << 2) + s) ^ key;
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) a[f] = *reinterpret_cast<const bf16x8_t*>(at + f * 32 * 128 + slot * 16);
#pragma unroll
      for (int g = 0; g < 2; ++g) b[g] = *reinterpret_cast<const bf16x8_t*>(bt + g * 32 * 128 + slot * 16);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f], b[g], acc[f][g], 0, 0, 0);
    }
  }

  // Epilogue through LDS, so that every global access is 16 bytes per lane along a row.  Register
  // r of a 32x32 accumulator tile holds row 8 (r / 4) + 4 hh + r % 4 and column lane % 32.
  // Staged rows are padded (fp32: 136 floats, bf16: 72) so that the two row groups a write
  // instruction touches (rows R and R + 4) fall in different banks.
  const int kChunks = C::kBM * 32 / C::kThreads;  // 16-byte fp32 chunks per thread
  float* out = static_cast<float*>(p.out);
  const bool vec = (p.N & 3) == 0;
  u32x4_t yv[C::kBM * 32 / C::kThreads];
  if constexpr (EPI == kEpiAccum) {
    // start reading the accumulated outputs while the tile is staged
    if (p.accumulate && vec) {
#pragma unroll
      for (int j = 0; j < kChunks; ++j) {
        const int i = threadIdx.x + j * C::kThreads, R = i >> 5, n = tn * kDBN + (i & 31) * 4;
        const int row = min(m0 + R, p.M - 1);
        if (n < p.N) yv[j] = *reinterpret_cast<const u32x4_t*>(out + (size_t)row * p.N + n);
      }
    }
  }
  __syncthreads();  // every wave is done reading the ring
  if constexpr (EPI == kEpiSwiglu) {
    constexpr int kS = 72;
    uint16_t* st = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = wm * 64 + f * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        st[R * kS + wn * 32 + m] = f32_to_bf16(silu_mul_f(acc[f][0][r], acc[f][1][r]));
      }
    __syncthreads();
    uint16_t* a_out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int j = 0; j < C::kBM * 8 / C::kThreads; ++j) {
      const int i = threadIdx.x + j * C::kThreads, R = i >> 3, c = i & 7;
      const int row = m0 + R, o = tn * 64 + c * 8;
      if (row < p.M && o < p.N)  // N is a multiple of 8: a chunk is all in or all out
        *reinterpret_cast<u32x4_t*>(a_out + (size_t)row * p.N + o) =
            *reinterpret_cast<const u32x4_t*>(st + R * kS + c * 8);
    }
  } else {
    constexpr int kS = 136;
    float* st = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int R = wm * 64 + f * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          st[R * kS + wn * 64 + g * 32 + m] = acc[f][g][r];
        }
    __syncthreads();
    const bool add = EPI == kEpiAccum && p.accumulate;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int i = threadIdx.x + j * C::kThreads, R = i >> 5, c = i & 31;
      const int row = m0 + R, n = tn * kDBN + c * 4;
      if (row >= p.M || n >= p.N) continue;
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(st + R * kS + c * 4);
      float* dst = out + (size_t)row * p.N + n;
      if (vec) {
        if (add) v += __builtin_bit_cast(f32x4_t, yv[j]);
        *reinterpret_cast<f32x4_t*>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) dst[e] = add ? dst[e] + v[e] : v[e];
      }
    }
  }
}

template <int WM, int EPI>
hipError_t launch_gemm(const DenseArgs& p, hipStream_t s) {
  using C = DenseCfg<WM>;
  const int nN = EPI == kEpiSwiglu ? (p.N + 63) / 64 : (p.N + kDBN - 1) / kDBN;
  const int nM = (p.M + C::kBM - 1) / C::kBM;
  const int lds = C::kNBuf * C::kStage;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dense_gemm_kernel<WM, EPI>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              DenseCfg<WM>::kNBuf * DenseCfg<WM>::kStage);
  });
  hipLaunchKernelGGL((dense_gemm_kernel<WM, EPI>), dim3(nM * nN), dim3(C::kThreads), lds, s, p);
  return hipGetLastError();
}

// Tiles of 256 rows when they still give at least one tile per CU, else 128.
template <int EPI>
hipError_t gemm(const DenseArgs& p, hipStream_t s) {
  const int nN = EPI == kEpiSwiglu ? (p.N + 63) / 64 : (p.N + kDBN - 1) / kDBN;
  if ((int64_t)((p.M + 255) / 256) * nN >= 256) return launch_gemm<4, EPI>(p, s);
  return launch_gemm<2, EPI>(p, s);
}

// ---------------------------------------------------------------------------------------------
// GEMV for M <= 8 token rows.  A workgroup of 256 threads covers 256 / LPR weight rows with LPR
// lanes each; lane c of a row multiplies 16-byte pieces c, c + LPR, ... of the row with the same
// pieces of every token row.  The first 16 pieces of the lane's row are requested before the
// token rows are staged in LDS, so the two latencies overlap.  The row's lanes then sum their
// partial dot products (shuffles within a wave, LDS across the waves of a row).  LPR is chosen
// per call so that the grid has about one workgroup per CU or more.

constexpr int kGemvMaxRows = 8;         // token rows the GEMV takes
constexpr int kGemvMaxLds = 64 * 1024;  // M * K * 2 bytes of staged token rows
constexpr int kGemvBatch = 16;          // pieces per lane requested ahead

STRATA_DEVICE float dot2_bf16(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, x), acc, false);
}

STRATA_DEVICE float dot8_bf16(const u32x4_t& w, const u32x4_t& x, float acc) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  return dot2_bf16(w.w, x.w, acc);
}

// TT >= M token rows; LDS holds TT staged rows (rows M .. TT - 1 are unset, their sums are never
// stored).  bid: this workgroup's index within the GEMV's grid.
template <int TT, int LPR, int EPI>
STRATA_DEVICE void gemv_body(const DenseArgs& p, int bid) {
  constexpr int RW = 256 / LPR;                  // weight rows per workgroup
  constexpr int WL = LPR < 64 ? LPR : 64;        // lanes of a row within one wave
  constexpr int WPR = LPR / WL;                  // waves per row
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, r = tid / LPR, c = tid % LPR;
  const int nk8 = p.K >> 3;  // 16-byte pieces per row
  const uint16_t* row;
  if constexpr (EPI == kEpiSwiglu) {  // rows 0 .. RW/2-1: gate, RW/2 .. RW-1: up, same outputs
    const int o = bid * (RW / 2) + r % (RW / 2);
    row = (r >= RW / 2 ? p.b1 : p.b0) + (size_t)min(o, p.N - 1) * p.K;
  } else {
    row = p.b0 + (size_t)min(bid * RW + r, p.N - 1) * p.K;
  }
  const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(row);
  u32x4_t w[kGemvBatch];
#pragma unroll
  for (int b = 0; b < kGemvBatch; ++b) {
    const int j = c + LPR * b;
    if (j < nk8) w[b] = __builtin_nontemporal_load(wrow + j);
  }
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p.a);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(lds);
    for (int i = tid; i < p.M * nk8; i += 256) dst[i] = src[i];
  }
  __syncthreads();
  const u32x4_t* xs = reinterpret_cast<const u32x4_t*>(lds);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  for (int j0 = 0;; j0 += LPR * kGemvBatch) {
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int j = j0 + c + LPR * b;
      if (j < nk8) {
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = dot8_bf16(w[b], xs[t * nk8 + j], acc[t]);
      }
    }
    if (j0 + LPR * kGemvBatch >= nk8) break;
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int j = j0 + LPR * kGemvBatch + c + LPR * b;
      if (j < nk8) w[b] = __builtin_nontemporal_load(wrow + j);
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
#pragma unroll
    for (int off = WL / 2; off >= 1; off >>= 1) acc[t] += __shfl_xor(acc[t], off, WL);
  }
  __syncthreads();  // the staged rows are no longer read: LDS now holds partial sums
  float* part = reinterpret_cast<float*>(lds);  // [RW][WPR][TT]
  if (c % WL == 0) {
#pragma unroll
    for (int t = 0; t < TT; ++t) part[(r * WPR + c / WL) * TT + t] = acc[t];
  }
  __syncthreads();
  auto total = [&](int rr, int t) {
    float v = part[rr * WPR * TT + t];
#pragma unroll
    for (int q = 1; q < WPR; ++q) v += part[(rr * WPR + q) * TT + t];
    return v;
  };
  if constexpr (EPI == kEpiSwiglu) {
    if (tid < (RW / 2) * TT) {
      const int o = tid / TT, t = tid % TT;
      const int n = bid * (RW / 2) + o;
      if (n < p.N && t < p.M)
        static_cast<uint16_t*>(p.out)[(size_t)t * p.N + n] =
            f32_to_bf16(silu_mul_f(total(o, t), total(o + RW / 2, t)));
    }
  } else {
    if (tid < RW * TT) {
      const int rr = tid / TT, t = tid % TT;
      const int n = bid * RW + rr;
      if (n < p.N && t < p.M) {
        float* out = static_cast<float*>(p.out) + (size_t)t * p.N + n;
        const float v = total(rr, t);
        if (EPI == kEpiAccum && p.accumulate) *out += v;
        else *out = v;
      }
    }
  }
}

template <int TT, int LPR, int EPI>
__global__ __launch_bounds__(256) void dense_gemv_kernel(DenseArgs p) {
  gemv_body<TT, LPR, EPI>(p, blockIdx.x);
}

// The router projection and the shared expert's gate/up projection in one launch (both read the
// same token rows): workgroups [0, g0) take the router rows, the rest the gate/up rows.
template <int TT, int LPR>
__global__ __launch_bounds__(256) void router_shared_up_kernel(DenseArgs router, DenseArgs up, int g0) {
  if ((int)blockIdx.x < g0) gemv_body<TT, LPR, kEpiStore>(router, blockIdx.x);
  else gemv_body<TT, LPR, kEpiSwiglu>(up, blockIdx.x - g0);
}

template <int TT, int LPR, int EPI>
hipError_t launch_gemv_t(const DenseArgs& p, hipStream_t s) {
  constexpr int RW = 256 / LPR;
  const int grid = EPI == kEpiSwiglu ? (p.N + RW / 2 - 1) / (RW / 2) : (p.N + RW - 1) / RW;
  const int lds = TT * p.K * 2 > 256 ? TT * p.K * 2 : 256;
  hipLaunchKernelGGL((dense_gemv_kernel<TT, LPR, EPI>), dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

template <int TT, int EPI>
hipError_t gemv_lpr(const DenseArgs& p, hipStream_t s) {
  // the fewest lanes per row that still give >= 256 workgroups and >= 2 pieces per lane
  const int rows = EPI == kEpiSwiglu ? 2 * p.N : p.N, nk8 = p.K / 8;
  if (rows / 8 >= 256 || nk8 < 128) return launch_gemv_t<TT, 32, EPI>(p, s);
  if (rows / 4 >= 256 || nk8 < 256) return launch_gemv_t<TT, 64, EPI>(p, s);
  return launch_gemv_t<TT, 128, EPI>(p, s);
}

template <int EPI>
hipError_t gemv(const DenseArgs& p, hipStream_t s) {
  if (p.M <= 1) return gemv_lpr<1, EPI>(p, s);
  if (p.M <= 2) return gemv_lpr<2, EPI>(p, s);
  if (p.M <= 4) return gemv_lpr<4, EPI>(p, s);
  return gemv_lpr<8, EPI>(p, s);
}

// Token rows the GEMV kernel for M rows is compiled for (LDS holds that many staged rows).
inline int gemv_rows(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

template <int EPI>
hipError_t dense(const DenseArgs& p, hipStream_t s) {
  if (p.M <= kGemvMaxRows && gemv_rows(p.M) * p.K * 2 <= kGemvMaxLds) return gemv<EPI>(p, s);
  return gemm<EPI>(p, s);
}

template <int TT, int LPR>
hipError_t launch_router_shared_up_t(const DenseArgs& r, const DenseArgs& u, hipStream_t s) {
  constexpr int RW = 256 / LPR;
  const int g0 = (r.N + RW - 1) / RW, g1 = (u.N + RW / 2 - 1) / (RW / 2);
  const int lds = TT * r.K * 2 > 256 ? TT * r.K * 2 : 256;
  hipLaunchKernelGGL((router_shared_up_kernel<TT, LPR>), dim3(g0 + g1), dim3(256), lds, s, r, u, g0);
  return hipGetLastError();
}

template <int TT>
hipError_t router_shared_up_lpr(const DenseArgs& r, const DenseArgs& u, hipStream_t s) {
  // as gemv_lpr, over the router's rows and the gate/up rows together
  const int rows = r.N + 2 * u.N, nk8 = r.K / 8;
  if (rows / 8 >= 256 || nk8 < 128) return launch_router_shared_up_t<TT, 32>(r, u, s);
  if (rows / 4 >= 256 || nk8 < 256) return launch_router_shared_up_t<TT, 64>(r, u, s);
  return launch_router_shared_up_t<TT, 128>(r, u, s);
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                                float* logits, hipStream_t s) {
  DenseArgs p{x, wr, nullptr, logits, T, E, H, 0};
  return dense<kEpiStore>(p, s);
}

bool router_shared_up_fits(int T, int H) {
  return T >= 1 && T <= kGemvMaxRows && gemv_rows(T) * H * 2 <= kGemvMaxLds;
}

hipError_t launch_router_shared_up(const uint16_t* x, const uint16_t* wr, int E, const uint16_t* wg,
                                   const uint16_t* wu, int Is, int T, int H, float* logits,
                                   uint16_t* a, hipStream_t s) {
  if (!router_shared_up_fits(T, H)) return hipErrorInvalidValue;
  DenseArgs r{x, wr, nullptr, logits, T, E, H, 0};
  DenseArgs u{x, wg, wu, a, T, Is, H, 0};
  if (T <= 1) return router_shared_up_lpr<1>(r, u, s);
  if (T <= 2) return router_shared_up_lpr<2>(r, u, s);
  if (T <= 4) return router_shared_up_lpr<4>(r, u, s);
  return router_shared_up_lpr<8>(r, u, s);
}

hipError_t launch_shared_expert(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                                const uint16_t* wd, int T, int H, int I, float* y, int accumulate,
                                uint16_t* a, hipStream_t s) {
  DenseArgs up{x, wg, wu, a, T, I, H, 0};
  hipError_t e = dense<kEpiSwiglu>(up, s);
  if (e != hipSuccess) return e;
  DenseArgs down{a, wd, nullptr, y, T, H, I, accumulate};
  return dense<kEpiAccum>(down, s);
}

}  // namespace strata
