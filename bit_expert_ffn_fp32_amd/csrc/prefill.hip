// Prefill path: grouped expert GEMMs on the matrix cores, combine, RMSNorm.
//
// The pages name the expert matrix multiply as the heaviest computation of the model and say the
// low-bit blocks are dequantized on the fly inside it ("Two-Day Port, 8x Faster Prefill: Strata
// Engine Benchmarked", Where Strata Is Fast); a larger prefill batch lets every expert's weights
// serve more tokens (same section).  Here every work unit is weight-stationary: one (expert,
// output slice) pair streams its packed 2- or 3-bit blocks once per chunk of up to 224 of the
// expert's tokens, decodes them in registers and feeds v_mfma_f32_32x32x16_f16 with fp32
// accumulation.
//
// Numerics.  A weight is d * (q - c0) with an fp16 scale d.  The decoder forms the fp16 product
// fp16(d * (q - c0)) with one round-to-nearest-even (exact whenever q - c0 = +-0.5; otherwise the
// product needs 12-13 significant bits and is rounded to fp16's 11).  Activations enter the
// matrix cores as fp16 (bf16 inputs convert exactly within fp16's normal range); the SiLU*mul
// intermediate is stored as fp16 and expert outputs as bf16.
//
// Operand order.  Within every group of 8 consecutive reduction indices the GEMM feeds the
// matrix cores the order P8 = {0,4,1,5,2,6,3,7}: the decoder then produces each fp16 pair from one
// byte-table lookup (v_perm_b32) in a per-block table of the four products fp16(d * (q - 1.5)).  The activations are stored in the same order (x by the
// conversion kernel, the intermediate by the up-projection epilogue), so the sums are unchanged.
//
// Work distribution.  Units (chunk, slice) are numbered so that the units of one expert are
// consecutive; blockIdx is mapped so that consecutive units run on the same XCD (workgroups are
// dealt to the 8 XCDs round-robin), which keeps an expert's weights and its tokens' activations
// in that XCD's L2 while all of its slices run.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace strata {

constexpr int kGemmThreads = 256;                 // 4 waves, one per SIMD
constexpr int kKS = 64;                           // reduction indices per pipeline stage (2 blocks)
constexpr int kFrags = kChunkRows / 32;           // 32-row fragments per chunk
constexpr int kWScaleBytes = 256 * 2 * 2;         // 256 weight rows x 2 fp16 scales per stage
constexpr int kLdsBudget = 150 * 1024;            // ring of stage buffers
constexpr size_t kGemmLds = kLdsBudget + kChunkRows * sizeof(int);

// Stage geometry of a unit with NF fragments: as many stage buffers as fit in the ring (the
// copies of all but the computed stage are in flight, hiding the ~2-3 us copy latency), capped
// so that the vector-memory counter can express the waits (at most 63 outstanding operations).
template <int FMT, int NF>
struct Pipe {
  static constexpr int kCB = FMT == 2 ? 8 : 12;
  static constexpr int kXBytes = NF * 32 * kKS * 2;         // activation tile
  static constexpr int kWCodeBytes = 4 * 128 * kCB;          // 4 weight tiles x 64 rows x 2 blocks
  static constexpr int kStage = kXBytes + kWCodeBytes + kWScaleBytes;
  static constexpr int kPer = NF + (FMT == 2 ? 1 : 2) + 1;   // copy instructions per wave per stage
  static constexpr int kByLds = kLdsBudget / kStage;
  static constexpr int kByCnt = 63 / kPer + 1;               // (buffers - 2) * kPer <= 63, with margin
  static constexpr int kNBuf = kByLds < kByCnt ? (kByLds < 8 ? kByLds : 8) : (kByCnt < 8 ? kByCnt : 8);
  static constexpr int kPD = kNBuf - 1;
  static_assert(kNBuf >= 2, "ring too small");
  static_assert((kPD - 1) * kPer <= 63, "vmcnt range");
};

STRATA_DEVICE int p8inv(int m) { return ((m & 3) << 1) | (m >> 2); }  // position of index m

// s_waitcnt with only the vector-memory counter constrained (at most N outstanding).
template <int N>
STRATA_DEVICE void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Waits until at most P later stages' copies are outstanding, for a runtime P in [0, PMAX].
template <int PER, int PMAX>
STRATA_DEVICE void wait_pending(int p) {
  if constexpr (PMAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (p >= PMAX) wait_vmcnt<PMAX * PER>();
    else wait_pending<PER, PMAX - 1>(p);
  }
}

// ---------------------------------------------------------------------------------------------
// Block decoders.  Per stage a lane owns one block (32 reduction indices) of each of its two
// weight rows and produces, for step s (0..3), the 8 fp16 weights of indices 8s .. 8s+7 of the
// block in P8 order.

struct Q2Tab {
  uint32_t lo, hi;  // byte q of lo/hi = low/high byte of fp16(d * (q - 1.5))
};

STRATA_DEVICE Q2Tab q2_table(uint16_t dbits) {
  const _Float16 d = __builtin_bit_cast(_Float16, dbits);
  const half2_t dd = {d, d};
  const half2_t p01 = dd * half2_t{(_Float16)-1.5f, (_Float16)-0.5f};  // one rounding each
  const half2_t p23 = dd * half2_t{(_Float16)0.5f, (_Float16)1.5f};
  const uint32_t u01 = __builtin_bit_cast(uint32_t, p01), u23 = __builtin_bit_cast(uint32_t, p23);
  return Q2Tab{__builtin_amdgcn_perm(u23, u01, 0x06040200u), __builtin_amdgcn_perm(u23, u01, 0x07050301u)};
}

// The selector constants of q2_decode, held in VGPRs so that each selector is one v_and_or_b32
// (gfx9 VOP3 takes no literal operand and reads at most one scalar register).
struct Q2Sel {
  uint32_t mask, base;
};

STRATA_DEVICE Q2Sel q2_sel() {
  Q2Sel k{0x03030303u, 0x04000400u};
  asm volatile("" : "+v"(k.mask), "+v"(k.base));
  return k;
}

// code: the block's 8 code bytes; bytes 2s, 2s+1 hold the codes of step s.
STRATA_DEVICE half8_t q2_decode(uint32_t w0, uint32_t w1, int s, const Q2Tab& tab, const Q2Sel& k) {
  const uint32_t word = (s >> 1) ? w1 : w0;
  const uint32_t X = __builtin_amdgcn_perm(word, word, (s & 1) ? 0x03030202u : 0x01010000u);
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sel = ((X >> (2 * i)) & k.mask) | k.base;
    r[i] = __builtin_amdgcn_perm(tab.hi, tab.lo, sel);
  }
  return __builtin_bit_cast(half8_t, r);
}

// 3-bit: the block's 12 code bytes as 3 words; step s covers bits 24s .. 24s+23.
STRATA_DEVICE half8_t q3_decode(uint32_t w0, uint32_t w1, uint32_t w2, int s, float d) {
  uint32_t v;
  if (s == 0) v = w0;
  else if (s == 1) v = __builtin_amdgcn_alignbit(w1, w0, 24);
  else if (s == 2) v = __builtin_amdgcn_alignbit(w2, w1, 16);
  else v = w2 >> 8;
  const float off = -3.5f * d;  // exact: 13 significant bits
  half8_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t qa = (v >> (3 * i)) & 7u, qb = (v >> (3 * i + 12)) & 7u;
    r[2 * i] = (_Float16)__builtin_fmaf((float)qa, d, off);  // exact in fp32, one rounding
    r[2 * i + 1] = (_Float16)__builtin_fmaf((float)qb, d, off);
  }
  return r;
}

// ---------------------------------------------------------------------------------------------
// Work units.

struct UnitInfo {
  int expert, row_start, nrows, nfrag, slice;
};

// Maps blockIdx to a unit; false if this workgroup has no unit.
STRATA_DEVICE bool pick_unit(const Chunk* chunks, const int* n_chunks, int n_slices, UnitInfo& u) {
  const int U = *n_chunks * n_slices;
  const int per = (U + 7) >> 3;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  if (i >= per) return false;
  const int unit = xcd * per + i;
  if (unit >= U) return false;
  const Chunk ch = chunks[unit / n_slices];
  u.expert = ch.expert;
  u.row_start = ch.row_start;
  u.nrows = ch.nrows;
  u.nfrag = (ch.nrows + 31) >> 5;
  u.slice = unit % n_slices;
  return true;
}

// ---------------------------------------------------------------------------------------------
// The K loop shared by both projections.
//
// Every stage (64 reduction indices) is copied global -> LDS by the workgroup with
// global_load_lds (lane i of a wave instruction lands at the instruction's LDS base + size*i):
//  * activation tile: NF*32 rows x 64 fp16 = 8 pieces of 16 B per row; piece c of row r sits in
//    slot c ^ (r % 8) so that a fragment read (8 consecutive rows, one piece each, per LDS cycle)
//    hits distinct banks; wave w copies the 8-row groups q = w, w+4, ...;
//  * weights: the unit's 256 rows are four 64-row weight tiles, one per wave; per stage a wave
//    copies its tile's codes (64 rows x 2 blocks, 1 or 1.5 KB) and scales (256 B) into the
//    tile's LDS slot as [64 rows][2 blocks][cb] and [64 rows][2] fp16.  In the tiled weight
//    layout those bytes are 16 contiguous pieces (one per 4-row group) of 64 / 96 bytes of codes
//    and 16 bytes of scales.
// Stages are issued kPD ahead into a ring of kNBuf buffers; each stage waits on the vector-memory
// counter for its own copies and a barrier makes them visible to all waves.

// This lane's stage-0 source addresses for the 64-row weight tile its wave copies.  Codes: lane l
// copies bytes 16 l .. 16 l + 15 of the tile's [64][2][cb] bytes (and, for 3-bit, l < 32 also
// 1024 + 16 l ..); scales: bytes 4 l .. 4 l + 3 of its [64][2] fp16.  Byte b of a tile-stage sits
// in 4-row group b / (8 cb) at offset b % (8 cb); successive stages of a group are 8 cb bytes
// (16 bytes of scales) apart.
struct WeightTile {
  const uint8_t* codes0;
  const uint8_t* codes1;
  const uint16_t* scales;
};

template <int FMT>
STRATA_DEVICE WeightTile weight_tile(const uint8_t* codes, const uint16_t* scales, size_t row0, int nkt) {
  constexpr int GB = 8 * (FMT == 2 ? 8 : 12);  // code bytes of one 4-row group stage
  const int lane = threadIdx.x & 63;
  const size_t g0 = row0 >> 2;
  const int b0 = lane * 16, b1 = 1024 + lane * 16;
  WeightTile wt;
  wt.codes0 = codes + (g0 + b0 / GB) * nkt * GB + b0 % GB;
  wt.codes1 = codes + (g0 + (FMT == 3 && lane < 32 ? b1 / GB : 0)) * nkt * GB + (FMT == 3 && lane < 32 ? b1 % GB : 0);
  wt.scales = scales + (g0 + (lane >> 2)) * nkt * 8 + (lane & 3) * 2;
  return wt;
}

// Copies c0 .. c1 - 1 of this wave's kPer copies of stage j: the NF activation groups, then the
// weight tile's codes (one or two), then its scales.
template <int FMT, int NF>
STRATA_DEVICE void issue_copies(uint8_t* stage, const uint16_t* __restrict__ src, const int (&xoff)[NF],
                                const WeightTile& wt, int j, int c0, int c1) {
  constexpr int TB = 128 * (FMT == 2 ? 8 : 12);  // code bytes of one 64-row tile-stage
  constexpr int GB = TB / 16;                     // code bytes of one 4-row group stage
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = j * kKS;
#pragma unroll
  for (int g = 0; g < NF; ++g) {
    if (g < c0 || g >= c1) continue;
    const int q = wave + 4 * g;
    __builtin_amdgcn_global_load_lds(src + xoff[g] + k0, stage + q * 1024, 16, 0, 0);
  }
  uint8_t* carea = stage + Pipe<FMT, NF>::kXBytes + wave * TB;
  if (NF >= c0 && NF < c1) __builtin_amdgcn_global_load_lds(wt.codes0 + (size_t)j * GB, carea, 16, 0, 0);
  constexpr int kS = NF + (FMT == 2 ? 1 : 2);  // index of the scale copy
  if constexpr (FMT == 3) {
    if (NF + 1 >= c0 && NF + 1 < c1 && lane < 32)
      __builtin_amdgcn_global_load_lds(wt.codes1 + (size_t)j * GB, carea + 1024, 16, 0, 0);
  }
  if (kS >= c0 && kS < c1)
    __builtin_amdgcn_global_load_lds(wt.scales + (size_t)j * 8,
                                     stage + Pipe<FMT, NF>::kXBytes + Pipe<FMT, NF>::kWCodeBytes + wave * 256, 4, 0, 0);
}

template <int FMT, int NF>
STRATA_DEVICE void issue_stage(uint8_t* stage, const uint16_t* __restrict__ src, const int (&xoff)[NF],
                               const WeightTile& wt, int j) {
  issue_copies<FMT, NF>(stage, src, xoff, wt, j, 0, Pipe<FMT, NF>::kPer);
}

// Per-lane weight state of one stage: the lane's block (hh) of its row in each stream (row ri of
// LDS weight tile ti) and what the decoder derives from the block scale.
template <int FMT>
struct StageWeights {
  uint32_t cw0[3], cw1[3];
  Q2Tab t0, t1;
  float f0, f1;
};

template <int FMT, int NF>
STRATA_DEVICE void load_stage_weights(StageWeights<FMT>& sw, const uint8_t* stage, int ti0, int ti1,
                                      int ri0, int ri1, int hh) {
  using P = Pipe<FMT, NF>;
  constexpr int CB = P::kCB;
  const uint8_t* carea = stage + P::kXBytes;
  const uint16_t* sarea = reinterpret_cast<const uint16_t*>(stage + P::kXBytes + P::kWCodeBytes);
  const uint32_t* p0 = reinterpret_cast<const uint32_t*>(carea + ti0 * 128 * CB + ri0 * 2 * CB + hh * CB);
  const uint32_t* p1 = reinterpret_cast<const uint32_t*>(carea + ti1 * 128 * CB + ri1 * 2 * CB + hh * CB);
  if constexpr (FMT == 2) {
    const uint2 v0 = *reinterpret_cast<const uint2*>(p0), v1 = *reinterpret_cast<const uint2*>(p1);
    sw.cw0[0] = v0.x; sw.cw0[1] = v0.y; sw.cw1[0] = v1.x; sw.cw1[1] = v1.y;
    sw.cw0[2] = sw.cw1[2] = 0;
  } else {
    sw.cw0[0] = p0[0]; sw.cw0[1] = p0[1]; sw.cw0[2] = p0[2];
    sw.cw1[0] = p1[0]; sw.cw1[1] = p1[1]; sw.cw1[2] = p1[2];
  }
  const uint16_t d0 = sarea[ti0 * 128 + ri0 * 2 + hh], d1 = sarea[ti1 * 128 + ri1 * 2 + hh];
  if constexpr (FMT == 2) {
    sw.t0 = q2_table(d0);
    sw.t1 = q2_table(d1);
  } else {
    sw.f0 = f16_to_f32(d0);
    sw.f1 = f16_to_f32(d1);
  }
}

// The B operands (both streams) of step s of the stage.
template <int FMT>
STRATA_DEVICE void decode_step(const StageWeights<FMT>& sw, int s, half8_t (&b)[2], const Q2Sel& k) {
  if constexpr (FMT == 2) {
    b[0] = q2_decode(sw.cw0[0], sw.cw0[1], s, sw.t0, k);
    b[1] = q2_decode(sw.cw1[0], sw.cw1[1], s, sw.t1, k);
  } else {
    b[0] = q3_decode(sw.cw0[0], sw.cw0[1], sw.cw0[2], s, sw.f0);
    b[1] = q3_decode(sw.cw1[0], sw.cw1[1], sw.cw1[2], s, sw.f1);
  }
}

// The A fragments of step s: row f*32 + m, 8 fp16 at piece (hh*4 + s) of the row.
template <int NF>
STRATA_DEVICE void read_frags(const uint8_t* xt, int m, int hh, int s, half8_t (&a)[NF]) {
  const int slot = ((hh << 2) + s) ^ ((m >> 1) & 7);
#pragma unroll
  for (int f = 0; f < NF; ++f)
    a[f] = *reinterpret_cast<const half8_t*>(xt + (f * 32 + m) * 128 + slot * 16);
}

template <int NF>
STRATA_DEVICE void mfma_step(f32x16_t (&acc0)[NF], f32x16_t (&acc1)[NF], const half8_t (&a)[NF],
                             const half8_t (&b)[2], int f0, int f1) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f < f0 || f >= f1) continue;
    acc0[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[f], b[0], acc0[f], 0, 0, 0);
    acc1[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[f], b[1], acc1[f], 0, 0, 0);
  }
}

// Software pipeline over the 4 steps of a stage: scheduling region s holds the matrix ops of step
// s together with the fragment reads and the weight decode of step s+1, so the decode's VALU work
// issues between the matrix ops.  The next stage's set-up (its barrier, weight words, decode
// tables, step-0 fragments and weights) runs inside step 3, behind the last matrix ops of this
// stage, so the matrix core does not wait for it at the stage boundary.
template <int FMT, int NF>
STRATA_DEVICE void gemm_core(f32x16_t (&acc0)[NF], f32x16_t (&acc1)[NF], const uint16_t* __restrict__ src,
                             int ld, int K, const int* rows_lds, const WeightTile& wt,
                             int ti0, int ti1, int ri0, int ri1, uint8_t* lds) {
  using P = Pipe<FMT, NF>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    acc0[f] = f32x16_t{};
    acc1[f] = f32x16_t{};
  }
  int xoff[NF];
#pragma unroll
  for (int g = 0; g < NF; ++g) {
    const int r = 8 * (wave + 4 * g) + (lane >> 3);
    xoff[g] = rows_lds[r] * ld + (((lane & 7) ^ ((r >> 1) & 7)) << 3);
  }
  const int NK = K / kKS;
#pragma unroll
  for (int j = 0; j < P::kPD; ++j)
    if (j < NK) issue_stage<FMT, NF>(lds + j * P::kStage, src, xoff, wt, j);
  // stage 0 landed for this wave (later stages may be outstanding), then for every wave.  Bare
  // s_barriers: __syncthreads() would also drain the copies in flight for the later stages.
  {
    const int later = NK - 1;
    wait_pending<P::kPer, P::kPD - 1>(later < P::kPD - 1 ? later : P::kPD - 1);
  }
  __builtin_amdgcn_s_barrier();
  const Q2Sel ksel = q2_sel();
  StageWeights<FMT> sw;
  half8_t a[2][NF];
  half8_t b[2][2];
  load_stage_weights<FMT, NF>(sw, lds, ti0, ti1, ri0, ri1, hh);
  read_frags<NF>(lds, m, hh, 0, a[0]);
  decode_step<FMT>(sw, 0, b[0], ksel);
  for (int j = 0; j < NK; ++j) {
    // stage j + kPD goes into the buffer of stage j - 1, which every wave finished reading before
    // the barrier that opened stage j.  Its copies are spread over steps 0-2, between the matrix
    // ops: a wave waits at a copy while the address unit still serves earlier ones, and the matrix
    // core keeps running meanwhile.  (All are issued before the wait in step 3, which counts them.)
    // Past the last stage the copies repeat stage NK - 1 into that free buffer, so that they stay
    // unconditional (no branch splits the step); the waits do not count them, which only makes
    // them stricter.
    const int jc = j + P::kPD < NK ? j + P::kPD : NK - 1;
    uint8_t* dst = lds + ((j + P::kPD) % P::kNBuf) * P::kStage;
    const uint8_t* xt = lds + (j % P::kNBuf) * P::kStage;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      issue_copies<FMT, NF>(dst, src, xoff, wt, jc, s * P::kPer / 3, (s + 1) * P::kPer / 3);
      read_frags<NF>(xt, m, hh, s + 1, a[(s + 1) & 1]);
      decode_step<FMT>(sw, s + 1, b[(s + 1) & 1], ksel);
      mfma_step<NF>(acc0, acc1, a[s & 1], b[s & 1], 0, NF);
    }
    __builtin_amdgcn_sched_barrier(0);
    // (on the last stage the set-up below reads a stale buffer; its results are not used.  It is
    // not skipped so that the step-3 matrix ops stay in one block with it.)
    {
      // the first matrix ops of step 3 keep the matrix core busy through the barrier
      constexpr int kPre = (NF + 1) / 2;
      mfma_step<NF>(acc0, acc1, a[1], b[1], 0, kPre);
      __builtin_amdgcn_sched_barrier(0);
      {
        const int later = NK - 2 - j;  // stages issued after stage j + 1
        wait_pending<P::kPer, P::kPD - 1>(later < 0 ? 0 : later < P::kPD - 1 ? later : P::kPD - 1);
      }
      // this wave's reads of stage j are complete before any wave may overwrite its buffer
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt / expcnt unconstrained
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* nt = lds + ((j + 1) % P::kNBuf) * P::kStage;
      load_stage_weights<FMT, NF>(sw, nt, ti0, ti1, ri0, ri1, hh);
      read_frags<NF>(nt, m, hh, 0, a[0]);
      decode_step<FMT>(sw, 0, b[0], ksel);
      mfma_step<NF>(acc0, acc1, a[1], b[1], kPre, NF);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // every wave is done with the stage buffers before the epilogue reuses them
}

// Row of a 32x32 accumulator tile held in register r of this lane.
STRATA_DEVICE int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

STRATA_DEVICE float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------------------------------------
// Up projection: A[p][n] = SiLU(x_t . W_g[n]) * (x_t . W_u[n]) for the chunk's rows p.
// Slice = 128 outputs; wave w owns outputs slice*128 + w*32 + (lane % 32), gate and up.

constexpr int kUpOutRow = 128 + 8;   // halfs per LDS row of the staged output tile
constexpr int kDownOutRow = 256;     // 224 rows x 256 halfs fit in the stage ring

template <int FMT, int NF>
STRATA_DEVICE void up_unit(const UnitInfo& u, const uint16_t* __restrict__ x16, const WeightTile& wt,
                           int H, int I, uint16_t* __restrict__ a16, uint8_t* lds_bytes,
                           const int* rows_lds) {
  f32x16_t accg[NF], accu[NF];
  // LDS weight tiles 0, 1 = gate rows 0-63, 64-127 of the slice; 2, 3 = the same up rows
  const int w = threadIdx.x >> 6, ri = (w & 1) * 32 + (threadIdx.x & 31);
  gemm_core<FMT, NF>(accg, accu, x16, H, H, rows_lds, wt, w >> 1, 2 + (w >> 1), ri, ri, lds_bytes);
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_bytes);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  // stage SiLU(g)*u as fp16 in LDS (columns in P8 order within groups of 8), then 16-byte stores
  const int lcol = wave * 32 + (nl & ~7) + p8inv(nl & 7);
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = f * 32 + acc_row(r, hh);
      lds[row * kUpOutRow + lcol] =
          __builtin_bit_cast(uint16_t, f32_to_f16_sat(silu_mul(accg[f][r], accu[f][r])));
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2 * NF; ++i) {
    const int p = threadIdx.x + i * kGemmThreads;  // 16 pieces per row
    const int r = p >> 4, c = p & 15;
    if (r < u.nrows)
      *reinterpret_cast<u32x4_t*>(a16 + (size_t)(u.row_start + r) * I + u.slice * 128 + c * 8) =
          *reinterpret_cast<const u32x4_t*>(lds + r * kUpOutRow + c * 8);
  }
}

template <int FMT>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_up_kernel(
    const uint16_t* __restrict__ x16, const int* __restrict__ sorted_slot, int k,
    const Chunk* __restrict__ chunks, const int* __restrict__ n_chunks,
    const uint8_t* __restrict__ gate_codes, const uint8_t* __restrict__ up_codes,
    const uint16_t* __restrict__ gate_scales, const uint16_t* __restrict__ up_scales, int H, int I,
    uint16_t* __restrict__ a16) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* rows_lds = reinterpret_cast<int*>(smem + kLdsBudget);
  UnitInfo u;
  if (!pick_unit(chunks, n_chunks, I / 128, u)) return;
  const int wave = threadIdx.x >> 6;
  // wave w copies gate (w < 2) or up rows 128 slice + 64 (w & 1) .. + 63 of the expert
  const size_t row0 = (size_t)u.expert * I + 128 * u.slice + 64 * (wave & 1);
  const WeightTile wt = weight_tile<FMT>(wave < 2 ? gate_codes : up_codes,
                                         wave < 2 ? gate_scales : up_scales, row0, H / 64);
  for (int r = threadIdx.x; r < u.nfrag * 32; r += kGemmThreads)
    rows_lds[r] = sorted_slot[u.row_start + (r < u.nrows ? r : 0)] / k;
  __syncthreads();
  switch (u.nfrag) {
    case 1: up_unit<FMT, 1>(u, x16, wt, H, I, a16, smem, rows_lds); break;
    case 2: up_unit<FMT, 2>(u, x16, wt, H, I, a16, smem, rows_lds); break;
    case 3: up_unit<FMT, 3>(u, x16, wt, H, I, a16, smem, rows_lds); break;
    case 4: up_unit<FMT, 4>(u, x16, wt, H, I, a16, smem, rows_lds); break;
    case 5: up_unit<FMT, 5>(u, x16, wt, H, I, a16, smem, rows_lds); break;
    case 6: up_unit<FMT, 6>(u, x16, wt, H, I, a16, smem, rows_lds); break;
    default: up_unit<FMT, 7>(u, x16, wt, H, I, a16, smem, rows_lds); break;
  }
}

// ---------------------------------------------------------------------------------------------
// Down projection: out[slot(p)][h] = A[p] . W_d[h] for the chunk's rows p, written as bf16 in
// slot order.  Slice = 256 outputs; wave w owns h = slice*256 + w*64 + nf*32 + (lane % 32).

template <int FMT, int NF>
STRATA_DEVICE void down_unit(const UnitInfo& u, const uint16_t* __restrict__ a16,
                             const int* __restrict__ sorted_slot, const WeightTile& wt, int H,
                             int I, uint16_t* __restrict__ expert_out, uint8_t* lds_bytes,
                             const int* rows_lds) {
  f32x16_t acc0[NF], acc1[NF];
  // LDS weight tile w = rows 64 w .. 64 w + 63 of the slice
  const int w = threadIdx.x >> 6, ri = threadIdx.x & 31;
  gemm_core<FMT, NF>(acc0, acc1, a16, I, I, rows_lds, wt, w, w, ri, 32 + ri, lds_bytes);
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_bytes);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = f * 32 + acc_row(r, hh);
      lds[row * kDownOutRow + wave * 64 + nl] = f32_to_bf16(acc0[f][r]);
      lds[row * kDownOutRow + wave * 64 + 32 + nl] = f32_to_bf16(acc1[f][r]);
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4 * NF; ++i) {
    const int p = threadIdx.x + i * kGemmThreads;  // 32 pieces per row
    const int r = p >> 5, c = p & 31;
    if (r < u.nrows) {
      const size_t slot = (size_t)sorted_slot[u.row_start + r];
      *reinterpret_cast<u32x4_t*>(expert_out + slot * H + u.slice * 256 + c * 8) =
          *reinterpret_cast<const u32x4_t*>(lds + r * kDownOutRow + c * 8);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_down_kernel(
    const uint16_t* __restrict__ a16, const int* __restrict__ sorted_slot,
    const Chunk* __restrict__ chunks, const int* __restrict__ n_chunks,
    const uint8_t* __restrict__ down_codes, const uint16_t* __restrict__ down_scales, int H, int I,
    uint16_t* __restrict__ expert_out) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* rows_lds = reinterpret_cast<int*>(smem + kLdsBudget);
  UnitInfo u;
  if (!pick_unit(chunks, n_chunks, H / 256, u)) return;
  const int wave = threadIdx.x >> 6;
  // wave w copies rows 256 slice + 64 w .. + 63 of the expert
  const size_t row0 = (size_t)u.expert * H + 256 * u.slice + 64 * wave;
  const WeightTile wt = weight_tile<FMT>(down_codes, down_scales, row0, I / 64);
  for (int r = threadIdx.x; r < u.nfrag * 32; r += kGemmThreads)
    rows_lds[r] = u.row_start + (r < u.nrows ? r : 0);
  __syncthreads();
  switch (u.nfrag) {
    case 1: down_unit<FMT, 1>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
    case 2: down_unit<FMT, 2>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
    case 3: down_unit<FMT, 3>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
    case 4: down_unit<FMT, 4>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
    case 5: down_unit<FMT, 5>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
    case 6: down_unit<FMT, 6>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
    default: down_unit<FMT, 7>(u, a16, sorted_slot, wt, H, I, expert_out, smem, rows_lds); break;
  }
}

// ---------------------------------------------------------------------------------------------
// x bf16 -> fp16 in P8 order (one thread per 8 values).

__global__ void x_to_f16_kernel(const uint16_t* __restrict__ x, size_t n8, uint16_t* __restrict__ x16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u32x4_t v = reinterpret_cast<const u32x4_t*>(x)[i];
  uint16_t in[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    in[2 * m] = (uint16_t)(v[m] & 0xFFFFu);
    in[2 * m + 1] = (uint16_t)(v[m] >> 16);
  }
  constexpr int P8[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  u32x4_t o;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, f32_to_f16_sat(bf16_to_f32(in[P8[2 * m]])));
    const uint32_t hi = __builtin_bit_cast(uint16_t, f32_to_f16_sat(bf16_to_f32(in[P8[2 * m + 1]])));
    o[m] = lo | (hi << 16);
  }
  reinterpret_cast<u32x4_t*>(x16)[i] = o;
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t][h] (+)= sum_j w[t][j] * out[t*k + j][h], j ascending (one thread per 8 h).

__global__ void combine_kernel(const uint16_t* __restrict__ out, const float* __restrict__ w, int T,
                               int k, int H, float* __restrict__ y, int accumulate) {
  const int h8 = H / 8;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * h8) return;
  const int t = (int)(i / h8), c = (int)(i % h8);
  float acc[8];
  if (accumulate) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(y + (size_t)t * H + c * 8)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(y + (size_t)t * H + c * 8)[1];
#pragma unroll
    for (int m = 0; m < 4; ++m) { acc[m] = a[m]; acc[m + 4] = b[m]; }
  }
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(out + ((size_t)t * k + j) * H + c * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[2 * m] = __builtin_fmaf(wj, __uint_as_float(v[m] << 16), s[2 * m]);
      s[2 * m + 1] = __builtin_fmaf(wj, __uint_as_float(v[m] & 0xFFFF0000u), s[2 * m + 1]);
    }
  }
  f32x4_t o0, o1;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    o0[m] = accumulate ? acc[m] + s[m] : s[m];
    o1[m] = accumulate ? acc[m + 4] + s[m + 4] : s[m + 4];
  }
  reinterpret_cast<f32x4_t*>(y + (size_t)t * H + c * 8)[0] = o0;
  reinterpret_cast<f32x4_t*>(y + (size_t)t * H + c * 8)[1] = o1;
}

// ---------------------------------------------------------------------------------------------
// RMSNorm (unit gain): one workgroup of 256 threads per row.

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int H, float eps,
                                                      uint16_t* __restrict__ x) {
  __shared__ float part[4];
  const float* row = h + (size_t)blockIdx.x * H;
  float ss = 0.0f;
  for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
    ss = __builtin_fmaf(v[0], v[0], ss);
    ss = __builtin_fmaf(v[1], v[1], ss);
    ss = __builtin_fmaf(v[2], v[2], ss);
    ss = __builtin_fmaf(v[3], v[3], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* xr = x + (size_t)blockIdx.x * H;
  for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
    const uint32_t lo = f32_to_bf16(v[0] * inv) | ((uint32_t)f32_to_bf16(v[1] * inv) << 16);
    const uint32_t hi = f32_to_bf16(v[2] * inv) | ((uint32_t)f32_to_bf16(v[3] * inv) << 16);
    *reinterpret_cast<uint2*>(xr + i) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------------------------
// Launchers

static int grid_for_units(int64_t max_units) { return (int)(8 * ((max_units + 7) / 8)); }

// The GEMM kernels use more than 64 KB of dynamic LDS; allow it once per process.
static void allow_big_lds() {
  static std::once_flag once;
  std::call_once(once, [] {
    const void* ks[4] = {reinterpret_cast<const void*>(ffn_up_kernel<2>),
                         reinterpret_cast<const void*>(ffn_up_kernel<3>),
                         reinterpret_cast<const void*>(ffn_down_kernel<2>),
                         reinterpret_cast<const void*>(ffn_down_kernel<3>)};
    for (const void* k : ks)
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
  });
}

hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, hipStream_t s) {
  const size_t n8 = (size_t)T * H / 8;
  x_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, x16);
  return hipGetLastError();
}

hipError_t launch_ffn_up(int fmt, const uint16_t* x16, const int* sorted_slot, int k,
                         const Chunk* chunks, const int* n_chunks, int max_chunks_,
                         const void* gate_codes, const void* up_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, int E, int H, int I, uint16_t* a16,
                         hipStream_t s) {
  (void)E;
  const int grid = grid_for_units((int64_t)max_chunks_ * (I / 128));
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  if (fmt == 2) {
    allow_big_lds();
    ffn_up_kernel<2><<<grid, kGemmThreads, kGemmLds, s>>>(x16, sorted_slot, k, chunks, n_chunks, gc,
                                                          uc, gate_scales, up_scales, H, I, a16);
  } else {
    allow_big_lds();
    ffn_up_kernel<3><<<grid, kGemmThreads, kGemmLds, s>>>(x16, sorted_slot, k, chunks, n_chunks, gc,
                                                          uc, gate_scales, up_scales, H, I, a16);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(int fmt, const uint16_t* a16, const int* sorted_slot,
                           const Chunk* chunks, const int* n_chunks, int max_chunks_,
                           const void* down_codes, const uint16_t* down_scales, int E, int H,
                           int I, uint16_t* expert_out, hipStream_t s) {
  (void)E;
  const int grid = grid_for_units((int64_t)max_chunks_ * (H / 256));
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  if (fmt == 2) {
    allow_big_lds();
    ffn_down_kernel<2><<<grid, kGemmThreads, kGemmLds, s>>>(a16, sorted_slot, chunks, n_chunks, dc,
                                                            down_scales, H, I, expert_out);
  } else {
    allow_big_lds();
    ffn_down_kernel<3><<<grid, kGemmThreads, kGemmLds, s>>>(a16, sorted_slot, chunks, n_chunks, dc,
                                                            down_scales, H, I, expert_out);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* expert_out, const float* w, int T, int k, int H, float* y,
                          int accumulate, hipStream_t s) {
  const size_t n = (size_t)T * (H / 8);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(expert_out, w, T, k, H, y, accumulate);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, int T, int H, float eps, uint16_t* x, hipStream_t s) {
  rmsnorm_kernel<<<T, 256, 0, s>>>(h, H, eps, x);
  return hipGetLastError();
}

}  // namespace strata
