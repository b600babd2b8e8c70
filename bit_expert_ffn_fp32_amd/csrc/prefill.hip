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
// fp16(d * 2^s * (q - c0)) with one round-to-nearest-even (exact whenever q - c0 = +-0.5;
// otherwise the product needs 12-13 significant bits and is rounded to fp16's 11), where the
// matrix's shift s (from the per-expert range statistics) puts its largest product in
// [2^14, 2^15): no scale overflows fp16 and blocks within 2^28 of the largest stay normal.
// Activations enter the matrix cores as fp16 scaled per token by 2^sx (the row's largest |x| in
// [2^14, 2^15), so the bf16 values convert exactly).  The SiLU*mul intermediate is stored as fp16
// scaled per row by the power of two that puts its Cauchy-Schwarz bound (|x| times the largest
// gate-row and up-row norms) just below 2^15, and the expert outputs as bf16.  Every power of two
// is taken back out exactly (ldexp) in the fp32 epilogues.
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
#include "strata_moe.h"
#include "topk.hpp"

namespace strata {

constexpr int kGemmThreads = 256;                 // 4 waves, one per SIMD
constexpr int kKS = 64;                           // reduction indices per pipeline stage (2 blocks)
constexpr int kFrags = kChunkRows / 32;           // 32-row fragments per chunk
constexpr int kWScaleBytes = 256 * 2 * 2;         // 256 weight rows x 2 fp16 scales per stage
constexpr int kGemmLds = 160 * 1024;              // the whole LDS of a CU
constexpr int kGemmLdsSmall = 80 * 1024;          // half of it: two small-fragment workgroups per CU
constexpr int kRowsBytes = 2 * kChunkRows * 4;    // a unit's source and destination rows
// Output staging: a 32-row region per wave (one fragment at a time) with padded rows.
constexpr int kUpOutRow = 32 + 8;                 // halfs per row: a wave's 32 outputs
constexpr int kDownOutRow = 64 + 8;               // halfs per row: a wave's 64 outputs
constexpr int kUpEpiBytes = 4 * 32 * kUpOutRow * 2;
constexpr int kDownEpiBytes = 4 * 32 * kDownOutRow * 2;

// Byte layout of one stage buffer of a unit with NF fragments.
template <int FMT, int NF>
struct Geom {
  static constexpr int kCB = FMT == 2 ? 8 : 12;
  static constexpr int kXBytes = NF * 32 * kKS * 2;         // activation tile
  static constexpr int kWCodeBytes = 4 * 128 * kCB;          // 4 weight tiles x 64 rows x 2 blocks
  static constexpr int kStage = kXBytes + kWCodeBytes + kWScaleBytes;
  static constexpr int kPer = NF + (FMT == 2 ? 1 : 2) + 1;   // copy instructions per wave per stage
};

// The stage ring in RING bytes: as many buffers as fit (the copies of all but the computed stage
// are in flight, hiding the ~2-3 us copy latency), capped so that the vector-memory counter can
// express the waits (at most 63 outstanding).
template <int FMT, int NF, int RING>
struct Pipe : Geom<FMT, NF> {
  using G = Geom<FMT, NF>;
  static constexpr int kByLds = RING / G::kStage;
  static constexpr int kByCnt = 63 / G::kPer + 1;            // (buffers - 2) * kPer <= 63, with margin
  static constexpr int kNBuf = kByLds < kByCnt ? (kByLds < 8 ? kByLds : 8) : (kByCnt < 8 ? kByCnt : 8);
  static constexpr int kPD = kNBuf - 1;
  static_assert(kNBuf >= 2, "ring too small");
  static_assert((kPD - 1) * G::kPer <= 63, "vmcnt range");
};

STRATA_DEVICE int p8inv(int m) { return ((m & 3) << 1) | (m >> 2); }  // position of index m

// s_waitcnt with only the vector-memory counter constrained (at most N outstanding).
template <int N>
STRATA_DEVICE void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) for a runtime n in [LO, HI] (a binary tree of uniform branches).
template <int LO, int HI>
STRATA_DEVICE void wait_vmcnt_range(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vmcnt_range<MID, HI>(n);
    else wait_vmcnt_range<LO, MID - 1>(n);
  }
}

// Waits until at most n vector-memory operations are outstanding (n clamped to [0, 63]).
STRATA_DEVICE void wait_vmcnt_dyn(int n) { wait_vmcnt_range<0, 63>(n < 0 ? 0 : n > 63 ? 63 : n); }

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

// sh: the matrix's range shift (at most 15 for this format): the products are d times the code
// offsets q - 1.5 scaled by 2^sh, which are exact fp16 constants (exponent field + sh), so each
// entry is fp16(d 2^sh (q - 1.5)) with one rounding and no extra operation per block.
STRATA_DEVICE Q2Tab q2_table(uint16_t dbits, int sh) {
  const uint32_t e = (uint32_t)sh << 10;
  const half2_t c01 = __builtin_bit_cast(half2_t, ((0xBE00u + e) & 0xFFFFu) | ((0xB800u + e) << 16));
  const half2_t c23 = __builtin_bit_cast(half2_t, ((0x3800u + e) & 0xFFFFu) | ((0x3E00u + e) << 16));
  const _Float16 d = __builtin_bit_cast(_Float16, dbits);
  const half2_t dd = {d, d};
  const half2_t p01 = dd * c01;  // one rounding each
  const half2_t p23 = dd * c23;
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

// 3-bit: the block's 12 code bytes as 3 words; step s covers bits 24s .. 24s+23.  A code q is
// placed in the mantissa of an fp16 2.0, giving 2 + q/4; minus 2.875 that is (q - 3.5)/4 exactly,
// and times 4d (exact: a power-of-two multiple of the scale) it is d (q - 3.5) with one rounding,
// so each pair costs a few bit operations and two packed fp16 operations.  d4: 4d in both halves.
STRATA_DEVICE half8_t q3_decode(uint32_t w0, uint32_t w1, uint32_t w2, int s, half2_t d4) {
  uint32_t v;
  if (s == 0) v = w0;
  else if (s == 1) v = __builtin_amdgcn_alignbit(w1, w0, 24);
  else if (s == 2) v = __builtin_amdgcn_alignbit(w2, w1, 16);
  else v = w2 >> 8;
  const half2_t off = {(_Float16)-2.875f, (_Float16)-2.875f};
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = v >> (3 * i);  // code a at bits 0..2, code b at bits 12..14
    const uint32_t h = ((t & 7u) << 7) | ((t & 0x7000u) << 11) | 0x40004000u;  // 2 + q/4 each
    const half2_t w = (__builtin_bit_cast(half2_t, h) + off) * d4;
    r[i] = __builtin_bit_cast(uint32_t, w);
  }
  return __builtin_bit_cast(half8_t, r);
}

// ---------------------------------------------------------------------------------------------
// Work units.

struct UnitInfo {
  int expert, row_start, nrows, nfrag, slice0, nsl;
};

// Maps blockIdx to a unit (a chunk and G consecutive column slices of it); false if this
// workgroup has none.  The units of XCD x (blockIdx % 8, with the usual round-robin dispatch) are
// a contiguous range, so the slice groups of one chunk run side by side on one L2.  SMALL: the
// list is the small part, whose first n_chunks[2] chunks belong to the skinny GEMMs.
template <bool SMALL>
STRATA_DEVICE bool pick_unit(const Chunk* chunks, const int* n_chunks, int n_groups, int G,
                             UnitInfo& u) {
  const int skip = SMALL ? n_chunks[2] : 0;
  const int U = (*n_chunks - skip) * n_groups;
  const int per = (U + 7) >> 3;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  if (i >= per) return false;
  const int unit = xcd * per + i;
  if (unit >= U) return false;
  const Chunk ch = chunks[skip + unit / n_groups];
  u.expert = ch.expert;
  u.row_start = ch.row_start;
  u.nrows = ch.nrows;
  u.nfrag = (ch.nrows + 31) >> 5;
  u.slice0 = (unit % n_groups) * G;
  u.nsl = G;
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

// Copies c0 .. c1 - 1 of this wave's kPer copies of one stage: the NF activation groups (columns
// 64 ks .. 64 ks + 63 of the rows xoff), then the weight tile's codes (one or two), then its
// scales; woff / soff: byte / fp16 offsets of the stage's weight pieces from stage 0 of slice 0.
template <int FMT, int NF>
STRATA_DEVICE void issue_copies(uint8_t* stage, const uint16_t* __restrict__ src, const int* xoff,
                                const WeightTile& wt, int ks, size_t woff, size_t soff, int c0, int c1) {
  using GM = Geom<FMT, NF>;
  constexpr int TB = 128 * GM::kCB;  // code bytes of one 64-row tile-stage
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = ks * kKS;
#pragma unroll
  for (int g = 0; g < NF; ++g) {
    if (g < c0 || g >= c1) continue;
    const int q = wave + 4 * g;
    __builtin_amdgcn_global_load_lds(src + xoff[g] + k0, stage + q * 1024, 16, 0, 0);
  }
  uint8_t* carea = stage + GM::kXBytes + wave * TB;
  if (NF >= c0 && NF < c1) __builtin_amdgcn_global_load_lds(wt.codes0 + woff, carea, 16, 0, 0);
  constexpr int kS = NF + (FMT == 2 ? 1 : 2);  // index of the scale copy
  if constexpr (FMT == 3) {
    if (NF + 1 >= c0 && NF + 1 < c1 && lane < 32)
      __builtin_amdgcn_global_load_lds(wt.codes1 + woff, carea + 1024, 16, 0, 0);
  }
  if (kS >= c0 && kS < c1)
    __builtin_amdgcn_global_load_lds(wt.scales + soff, stage + GM::kXBytes + GM::kWCodeBytes + wave * 256, 4, 0, 0);
}

// Per-lane weight state of one stage: the lane's block (hh) of its row in each stream (row ri of
// LDS weight tile ti) and what the decoder derives from the block scale.
template <int FMT>
struct StageWeights {
  uint32_t cw0[3], cw1[3];
  Q2Tab t0, t1;
  half2_t d40, d41;  // 3-bit: 4 d of each stream's block, in both halves
};

template <int FMT, int NF>
STRATA_DEVICE void load_stage_weights(StageWeights<FMT>& sw, const uint8_t* stage, int ti0, int ti1,
                                      int ri0, int ri1, int hh, int sh0, int sh1) {
  using GM = Geom<FMT, NF>;
  constexpr int CB = GM::kCB;
  const uint8_t* carea = stage + GM::kXBytes;
  const uint16_t* sarea = reinterpret_cast<const uint16_t*>(stage + GM::kXBytes + GM::kWCodeBytes);
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
    sw.t0 = q2_table(d0, sh0);
    sw.t1 = q2_table(d1, sh1);
  } else {
    const _Float16 e0 = __builtin_ldexpf16(__builtin_bit_cast(_Float16, d0), sh0 + 2);  // 4 d 2^s
    const _Float16 e1 = __builtin_ldexpf16(__builtin_bit_cast(_Float16, d1), sh1 + 2);
    sw.d40 = half2_t{e0, e0};
    sw.d41 = half2_t{e1, e1};
  }
}

// The B operands (both streams) of step s of the stage.
template <int FMT>
STRATA_DEVICE void decode_step(const StageWeights<FMT>& sw, int s, half8_t (&b)[2], const Q2Sel& k) {
  if constexpr (FMT == 2) {
    b[0] = q2_decode(sw.cw0[0], sw.cw0[1], s, sw.t0, k);
    b[1] = q2_decode(sw.cw1[0], sw.cw1[1], s, sw.t1, k);
  } else {
    b[0] = q3_decode(sw.cw0[0], sw.cw0[1], sw.cw0[2], s, sw.d40);
    b[1] = q3_decode(sw.cw1[0], sw.cw1[1], sw.cw1[2], s, sw.d41);
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

// Row of a 32x32 accumulator tile held in register r of this lane.
STRATA_DEVICE int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// The stored intermediate fp16(2^es * SiLU(g) * u) from the fp32 sums acc_g = 2^-ecg g and
// acc_u of the scaled operands: SiLU(g) u 2^es = acc_g acc_u sigmoid(g) 2^es' with the row's
// shifts folded into es by the caller; below 2^15 by construction (clamped to fp16's range
// regardless).
STRATA_DEVICE _Float16 silu_mul_scaled(float acc_g, float acc_u, int ecg, int es) {
  const float g = __builtin_ldexpf(acc_g, ecg);
  const float v = acc_g * acc_u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  return (_Float16)__builtin_amdgcn_fmed3f(__builtin_ldexpf(v, es), -65504.0f, 65504.0f);
}

// Per-row exponents of a unit (one int per unit row, in LDS):
//  up:   ecg (low 16 bits, signed) = -(sx + shift_gate), taking the gate sum back to g;
//        es (high 16 bits, signed) = 15 - E with the row's bound n2 * norm_gate_up < 2^E;
//  down: -(es + 2 sx + shift_gate + shift_up + shift_down), taking the down sum back to out.
STRATA_DEVICE int a_exponent(const XInfo& xi, const strata_moe_expert_stats& st) {
  const float b = xi.n2 * st.norm_gate_up;
  return b > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(b) : 15;
}

template <bool UP>
STRATA_DEVICE int row_exponent(const XInfo& xi, const strata_moe_expert_stats& st) {
  const int es = a_exponent(xi, st);
  if constexpr (UP) return (int)((uint32_t)(-(xi.sx + st.shift_gate)) & 0xFFFFu) | (es << 16);
  else return -(es + 2 * xi.sx + st.shift_gate + st.shift_up + st.shift_down);
}

// Two fp32 values as a bf16 pair (low half a), each rounded to nearest even: one packed hardware
// conversion (the same rounding as f32_to_bf16 for finite values).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
STRATA_DEVICE uint32_t bf16_pair_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Writes one slice's outputs, fragment by fragment, with 16-byte stores through a private LDS region
// of each wave (the columns a wave computes are the columns it stores, so no wave waits for the
// others; a staging buffer shared by the four waves needed a workgroup barrier per fragment).  Up: out = A (fp16, [rows][I],
// columns in P8 order within groups of 8), 128 outputs per slice, wave w holding outputs
// 32 w + n (acc0 = gate, acc1 = up); down: out = expert outputs (bf16, [slots][H]), 256 per
// slice, wave w holding columns 64 w + n (acc0) and 64 w + 32 + n (acc1).  dst_lds[r]: the
// destination row of unit row r (rows past the chunk repeat row 0, whose values they equal, so
// every lane stores); exps[r]: its exponents (row_exponent).  Each wave issues kStores stores per
// fragment.
template <int NF, bool UP>
struct Epilogue {
  static constexpr int kCols = UP ? 32 : 64;                        // a wave's columns
  static constexpr int kRow = kCols + 8;                            // halfs per staged row
  static constexpr int kPieces = kCols / 8;                         // 16-byte pieces per row
  static constexpr int kStores = 32 * kPieces / kWave;              // per lane per fragment
  static constexpr int kRegion = 32 * kRow;                         // halfs per wave
};

template <int NF, bool UP>
STRATA_DEVICE void write_slice(f32x16_t (&acc0)[NF], f32x16_t (&acc1)[NF], uint16_t* epi,
                               const int* dst_lds, const int* exps, uint16_t* __restrict__ out,
                               int out_ld, int col0) {
  using EP = Epilogue<NF, UP>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  uint16_t* const wr = epi + wave * EP::kRegion;  // this wave's region
  // this lane's first staged element (tile row 4 hh, its column); register r of a tile adds
  // rows 8 (r >> 2) + (r & 3), a constant offset
  const int lcol = UP ? (nl & ~7) + p8inv(nl & 7) : nl;
  uint16_t* const e0 = wr + 4 * hh * EP::kRow + lcol;
  // (opaque to the optimizer, so that the store addresses are not computed once for every slice
  // and held in registers across the main loop)
  asm volatile("" : "+s"(out_ld));
  const int cw = col0 + wave * EP::kCols;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    // One fragment at a time: the empty asm re-defines this fragment's sums in the accumulation
    // registers here, so their copies into VGPRs cannot be hoisted above it (all fragments'
    // copies at once would need 32 NF VGPRs).
    asm volatile("" : "+a"(acc0[f]), "+a"(acc1[f]));
    // exponents of this lane's rows f*32 + 8 q + 4 hh + (0..3), q = r >> 2
    int ex[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int4 v = *reinterpret_cast<const int4*>(exps + f * 32 + 8 * q + 4 * hh);
      ex[4 * q] = v.x; ex[4 * q + 1] = v.y; ex[4 * q + 2] = v.z; ex[4 * q + 3] = v.w;
    }
    if constexpr (UP) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ecg = (int)(int16_t)(ex[r] & 0xFFFF), es = ex[r] >> 16;
        e0[(8 * (r >> 2) + (r & 3)) * EP::kRow] =
            __builtin_bit_cast(uint16_t, silu_mul_scaled(acc0[f][r], acc1[f][r], ecg, es));
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t b = bf16_pair_rne(__builtin_ldexpf(acc0[f][r], ex[r]), __builtin_ldexpf(acc1[f][r], ex[r]));
        e0[(8 * (r >> 2) + (r & 3)) * EP::kRow] = (uint16_t)b;
        e0[(8 * (r >> 2) + (r & 3)) * EP::kRow + 32] = (uint16_t)(b >> 16);
      }
    }
    // the wave's values are in place (a wave's LDS operations complete in order; the clobber keeps
    // the compiler from moving the reads above the writes)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < EP::kStores; ++i) {
      const int p = lane + i * kWave;
      const int r = p / EP::kPieces, c = p % EP::kPieces;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wr + r * EP::kRow + c * 8);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (size_t)dst_lds[f * 32 + r] * out_ld + cw + c * 8);
      if constexpr (UP) *dst = v;                         // a: read again by the down GEMM
      else __builtin_nontemporal_store(v, dst);           // expert outputs: read once, by the combine
    }
    // (the next fragment's writes come after these reads)
    asm volatile("" ::: "memory");
  }
}

// Pipeline state carried from one stage to the next: the lane's weight words and decode tables of
// the current stage, and the step-0 (even) / step-1.. operands.
template <int FMT, int NF>
struct StageState {
  StageWeights<FMT> sw;
  half8_t a[2][NF];
  half8_t b[2][2];
};

// Stage set-up: weight words and tables, step-0 fragments and weights of the stage in buffer st.
template <int FMT, int NF>
STRATA_DEVICE void stage_setup(StageState<FMT, NF>& ss, const uint8_t* st, int ti0, int ti1, int ri0,
                               int ri1, int sh0, int sh1, const Q2Sel& ksel) {
  const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
  load_stage_weights<FMT, NF>(ss.sw, st, ti0, ti1, ri0, ri1, hh, sh0, sh1);
  read_frags<NF>(st, m, hh, 0, ss.a[0]);
  decode_step<FMT>(ss.sw, 0, ss.b[0], ksel);
}

// Copy cursor of a unit: the next stage to copy as (reduction stage ks, weight offsets woff /
// soff from slice 0 stage 0), moving through the unit's NT stages, NKs per slice, and staying on
// the last one (whose copies then repeat).
struct CopyCursor {
  int j, ks, NT, NKs;
  size_t woff, soff, wslice, sslice;
};

template <int FMT>
STRATA_DEVICE void cursor_advance(CopyCursor& c) {
  constexpr int GB = 8 * (FMT == 2 ? 8 : 12);  // code bytes of a 4-row group stage
  if (c.j + 1 >= c.NT) return;
  ++c.j;
  if (++c.ks == c.NKs) {
    c.ks = 0;
    c.woff += c.wslice - (size_t)(c.NKs - 1) * GB;
    c.soff += c.sslice - (size_t)(c.NKs - 1) * 8;
  } else {
    c.woff += GB;
    c.soff += 8;
  }
}

// Steps 0-2 of the stage in buffer xt (set up by stage_setup), with the copies of the cursor's
// stage into dst spread between them, and the first PRE fragments of step 3.
template <int FMT, int NF, int PER, int PRE>
STRATA_DEVICE void stage_steps(f32x16_t (&acc0)[NF], f32x16_t (&acc1)[NF], StageState<FMT, NF>& ss,
                               const uint8_t* xt, const Q2Sel& ksel, uint8_t* dst,
                               const uint16_t* __restrict__ src, const int (&xoff)[NF],
                               const WeightTile& wt, const CopyCursor& cc) {
  const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    issue_copies<FMT, NF>(dst, src, xoff, wt, cc.ks, cc.woff, cc.soff, s * PER / 3, (s + 1) * PER / 3);
    read_frags<NF>(xt, m, hh, s + 1, ss.a[(s + 1) & 1]);
    decode_step<FMT>(ss.sw, s + 1, ss.b[(s + 1) & 1], ksel);
    mfma_step<NF>(acc0, acc1, ss.a[s & 1], ss.b[s & 1], 0, NF);
    // One wave per SIMD issues in order: spread the step's other instructions (copies, fragment
    // reads, decode) between its matrix ops, four after each, so that neither waits behind a
    // long run of the other.  (2-bit: T = 8192 expert FFN 819 -> 855 TFLOP/s; group sizes 3-8
    // measured, 4 best.  The 3-bit decode, with more VALU work per step, measured slower with
    // any group size and keeps the compiler's order.)
    if constexpr (FMT == 2) {
#pragma unroll
      for (int i = 0; i < 2 * NF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // a matrix op
        __builtin_amdgcn_sched_group_barrier(0x002 | 0x004 | 0x020 | 0x100, 4, 0);  // VALU, SALU, VMEM and DS reads
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma_step<NF>(acc0, acc1, ss.a[1], ss.b[1], 0, PRE);
  __builtin_amdgcn_sched_barrier(0);
}

// Vector-memory operations a wave issued after the copies of stage m, up to the wait for it: the
// copies of the later stages that exist (PER each, at most PD - 1 stages ahead) and the ST stores
// of each slice that ended at iterations m - PD .. e0 (e0: the latest slice end before the wait,
// -1 if none; slice ends are NKs apart).
template <int PER, int PD>
STRATA_DEVICE int ops_after(int m, int e0, int NT, int NKs, int ST) {
  int n = PER * max(0, min(PD - 1, NT - 1 - m));
  for (int e = e0; e >= 0 && e >= m - PD; e -= NKs) n += ST;
  return n;
}

// Stage-boundary wait: this wave's copies of the next stage have landed (n operations issued
// after them may still be outstanding) and its own LDS reads are complete; then every wave's.
// A bare s_barrier: __syncthreads() would also drain the copies in flight for later stages.
// STEADY: the usual n (kPD - 1 later stages, no stores), waited for without the branch tree.
template <int STEADY>
STRATA_DEVICE void stage_barrier(int n) {
  if (n == STEADY) wait_vmcnt<STEADY>();
  else wait_vmcnt_dyn(n);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt / expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// One unit: rows of a chunk times G consecutive column slices, as one pipeline of G * K/64
// stages (stage js: slice js / (K/64), reduction stage js % (K/64)).  A slice's outputs are
// written when its last stage is done, while the next slice's copies are already in flight.
//
// Software pipeline over the 4 steps of a stage: scheduling region s holds the matrix ops of step
// s together with the fragment reads and the weight decode of step s+1, so the decode's VALU work
// issues between the matrix ops.  Within a slice the next stage's set-up (its barrier, weight
// words, decode tables, step-0 fragments and weights) runs inside step 3, behind the last matrix
// ops of the stage, so the matrix core does not wait for it at the stage boundary.
//
// Copies: stage j + kPD goes into the buffer of stage j - 1, which every wave finished reading
// before the barrier that opened stage j; its copies are spread over steps 0-2, between the
// matrix ops (a wave waits at a copy while the address unit still serves earlier ones, and the
// matrix core keeps running meanwhile).  Past the last stage the copies repeat stage NT - 1 into
// that free buffer, so that they stay unconditional (no branch splits the step).  The waits count
// the copies and stores issued after the awaited stage's copies, except those repeats, which only
// makes them stricter.
//
// src/ld: the activation rows (rows_lds[r]: row of unit row r); wt: this lane's weight pieces of
// slice 0, stage 0; wslice / sslice: byte / fp16 distance between slices in the tiled weights;
// (ti, ri): this lane's B rows in the LDS weight tiles; sh0 / sh1: the range shifts of the two
// weight streams; out/out_ld/ocols: destination and the columns per slice.  tok: the token of
// unit row threadIdx.x (-1 past the unit's rows), whose range (xinfo) is copied into the
// epilogue staging area (unused until the first slice ends) with the first stage; st: the
// expert's range statistics.  Once every wave has taken its activation offsets from rows_lds,
// the rows' exponents (row_exponent) replace them there for the epilogues.
template <int FMT, int NF, bool UP, int LDSB>
STRATA_DEVICE void run_unit(const UnitInfo& u, const uint16_t* __restrict__ src, int ld, int K,
                            int* rows_lds, const int* dst_lds, const WeightTile& wt,
                            size_t wslice, size_t sslice, int ti0, int ti1, int ri0, int ri1,
                            int sh0, int sh1, const XInfo* __restrict__ xinfo, int tok,
                            const strata_moe_expert_stats& st, uint16_t* __restrict__ out,
                            int out_ld, int ocols, uint8_t* lds) {
  constexpr int kEpi = UP ? kUpEpiBytes : kDownEpiBytes;
  using P = Pipe<FMT, NF, LDSB - kRowsBytes - kEpi>;
  using EP = Epilogue<NF, UP>;
  constexpr int kSt = EP::kStores * NF;  // stores per wave per slice
  constexpr int kPre = (NF + 1) / 2;     // step-3 fragments issued before the stage barrier
  uint16_t* epi = reinterpret_cast<uint16_t*>(lds + P::kNBuf * P::kStage);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x16_t acc0[NF], acc1[NF];
  int xoff[NF];
#pragma unroll
  for (int g = 0; g < NF; ++g) {
    const int r = 8 * (wave + 4 * g) + (lane >> 3);
    xoff[g] = rows_lds[r] * ld + (((lane & 7) ^ ((r >> 1) & 7)) << 3);
  }
  const int NKs = K / kKS, NT = u.nsl * NKs;
  // the rows' token ranges: words sx at epi + 4 r, n2 at epi + 1024 + 4 r (copies without a
  // register result, so no wait lands before the first stage barrier)
  uint8_t* const xr = reinterpret_cast<uint8_t*>(epi);
  if (tok >= 0) {
    const int32_t* src_xi = reinterpret_cast<const int32_t*>(xinfo + tok);
    __builtin_amdgcn_global_load_lds(src_xi, xr + wave * 256, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(src_xi + 1, xr + 1024 + wave * 256, 4, 0, 0);
  }
  CopyCursor cc{0, 0, NT, NKs, 0, 0, wslice, sslice};
#pragma unroll
  for (int j = 0; j < P::kPD; ++j)
    if (j < NT) {
      issue_copies<FMT, NF>(lds + j * P::kStage, src, xoff, wt, cc.ks, cc.woff, cc.soff, 0, P::kPer);
      cursor_advance<FMT>(cc);
    }
  stage_barrier<P::kPer * (P::kPD - 1)>(ops_after<P::kPer, P::kPD>(0, -1, NT, NKs, kSt));
  // (every wave has read rows_lds; the stage barriers of the first slice order these writes
  // before the epilogue's reads)
  if ((int)threadIdx.x < NF * 32) {
    const XInfo xi{reinterpret_cast<const int32_t*>(xr)[threadIdx.x],
                   reinterpret_cast<const float*>(xr + 1024)[threadIdx.x]};
    rows_lds[threadIdx.x] = row_exponent<UP>(xi, st);
  }
  const Q2Sel ksel = q2_sel();
  StageState<FMT, NF> ss;
  stage_setup<FMT, NF>(ss, lds, ti0, ti1, ri0, ri1, sh0, sh1, ksel);
  int j = 0, rb = 0;  // stage and its ring buffer
  int last_end = -1;  // iteration of the latest slice end
  for (int sl = 0; sl < u.nsl; ++sl) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      acc0[f] = f32x16_t{};
      acc1[f] = f32x16_t{};
    }
    // the slice's stages; each sets up the next one (on the unit's last stage: a stale buffer,
    // whose results are not used) inside its step 3
    for (int ks = 0; ks < NKs; ++ks, ++j) {
      const int nb = rb + 1 == P::kNBuf ? 0 : rb + 1;                    // buffer of stage j + 1
      uint8_t* dst = lds + (rb == 0 ? P::kNBuf - 1 : rb - 1) * P::kStage;  // of stage j - 1
      stage_steps<FMT, NF, P::kPer, kPre>(acc0, acc1, ss, lds + rb * P::kStage, ksel, dst, src, xoff,
                                          wt, cc);
      cursor_advance<FMT>(cc);
      stage_barrier<P::kPer * (P::kPD - 1)>(ops_after<P::kPer, P::kPD>(j + 1, last_end, NT, NKs, kSt));
      // (the set-up writes the even operands; step 3 uses the odd ones)
      stage_setup<FMT, NF>(ss, lds + nb * P::kStage, ti0, ti1, ri0, ri1, sh0, sh1, ksel);
      mfma_step<NF>(acc0, acc1, ss.a[1], ss.b[1], kPre, NF);
      __builtin_amdgcn_sched_barrier(0);
      rb = nb;
    }
    // (the staging area is separate from the stage ring, which the next slice's copies fill)
    write_slice<NF, UP>(acc0, acc1, epi, dst_lds, rows_lds, out, out_ld, (u.slice0 + sl) * ocols);
    last_end = j - 1;
  }
}

// ---------------------------------------------------------------------------------------------
// Up projection: A[p][n] = SiLU(x_t . W_g[n]) * (x_t . W_u[n]) for the chunk's rows p.
// Slice = 128 outputs; wave w owns outputs slice*128 + w*32 + (lane % 32), gate and up.
//
// NFMAX: the most fragments a unit holds, 7 (chunks of up to 224 rows; one workgroup per CU with
// the whole LDS) or 2 (chunks of up to 64 rows; half the LDS and at most 256 registers a wave, so
// that two workgroups share a CU).

template <int FMT, int NFMAX>
__global__ __launch_bounds__(kGemmThreads, NFMAX <= 2 ? 2 : 1) void ffn_up_kernel(
    const uint16_t* __restrict__ x16, const XInfo* __restrict__ xinfo,
    const int* __restrict__ sorted_slot, int k, const Chunk* __restrict__ chunks,
    const int* __restrict__ n_chunks, const uint8_t* __restrict__ gate_codes,
    const uint8_t* __restrict__ up_codes, const uint16_t* __restrict__ gate_scales,
    const uint16_t* __restrict__ up_scales, const strata_moe_expert_stats* __restrict__ stats,
    int H, int I, int G, uint16_t* __restrict__ a16) {
  constexpr int LDSB = NFMAX <= 2 ? kGemmLdsSmall : kGemmLds;
  extern __shared__ __align__(16) uint8_t smem[];
  int* rows_lds = reinterpret_cast<int*>(smem + LDSB - kRowsBytes);
  int* dst_lds = rows_lds + kChunkRows;
  UnitInfo u;
  if (!pick_unit<NFMAX <= 2>(chunks, n_chunks, I / 128 / G, G, u)) return;
  constexpr int GB = 8 * (FMT == 2 ? 8 : 12);
  const int wave = threadIdx.x >> 6, nkt = H / 64;
  // wave w copies gate (w < 2) or up rows 128 slice + 64 (w & 1) .. + 63 of the expert
  const size_t row0 = (size_t)u.expert * I + 128 * u.slice0 + 64 * (wave & 1);
  const WeightTile wt = weight_tile<FMT>(wave < 2 ? gate_codes : up_codes,
                                         wave < 2 ? gate_scales : up_scales, row0, nkt);
  const strata_moe_expert_stats st = stats[u.expert];
  int tok = -1;
  if ((int)threadIdx.x < u.nfrag * 32) {  // one unit row per thread (at most 224)
    const int r = threadIdx.x, rr = r < u.nrows ? r : 0;
    tok = sorted_slot[u.row_start + rr] / k;
    rows_lds[r] = tok;
    dst_lds[r] = u.row_start + rr;
  }
  __syncthreads();
  // a slice is 128 gate (and up) rows = 32 groups of 4
  const size_t wsl = (size_t)32 * nkt * GB, ssl = (size_t)32 * nkt * 8;
  // LDS weight tiles 0, 1 = gate rows 0-63, 64-127 of the slice; 2, 3 = the same up rows
  const int ri = (wave & 1) * 32 + (threadIdx.x & 31);
#define STRATA_UP_UNIT(NF)                                                                        \
  run_unit<FMT, NF, true, LDSB>(u, x16, H, H, rows_lds, dst_lds, wt, wsl, ssl, wave >> 1,           \
                                2 + (wave >> 1), ri, ri, st.shift_gate, st.shift_up, xinfo, tok, st, \
                                a16, I, 128, smem)
  if constexpr (NFMAX <= 2) {
    if (u.nfrag == 1) STRATA_UP_UNIT(1);
    else STRATA_UP_UNIT(2);
  } else {
    switch (u.nfrag) {
      case 1: STRATA_UP_UNIT(1); break;
      case 2: STRATA_UP_UNIT(2); break;
      case 3: STRATA_UP_UNIT(3); break;
      case 4: STRATA_UP_UNIT(4); break;
      case 5: STRATA_UP_UNIT(5); break;
      case 6: STRATA_UP_UNIT(6); break;
      default: STRATA_UP_UNIT(7); break;
    }
  }
#undef STRATA_UP_UNIT
}

// ---------------------------------------------------------------------------------------------
// Down projection: out[slot(p)][h] = A[p] . W_d[h] for the chunk's rows p, written as bf16 in
// slot order.  Slice = 256 outputs; wave w owns h = slice*256 + w*64 + nf*32 + (lane % 32).

template <int FMT, int NFMAX>
__global__ __launch_bounds__(kGemmThreads, NFMAX <= 2 ? 2 : 1) void ffn_down_kernel(
    const uint16_t* __restrict__ a16, const XInfo* __restrict__ xinfo,
    const int* __restrict__ sorted_slot, int k, const Chunk* __restrict__ chunks,
    const int* __restrict__ n_chunks, const uint8_t* __restrict__ down_codes,
    const uint16_t* __restrict__ down_scales, const strata_moe_expert_stats* __restrict__ stats,
    int H, int I, int G, uint16_t* __restrict__ expert_out) {
  constexpr int LDSB = NFMAX <= 2 ? kGemmLdsSmall : kGemmLds;
  extern __shared__ __align__(16) uint8_t smem[];
  int* rows_lds = reinterpret_cast<int*>(smem + LDSB - kRowsBytes);
  int* dst_lds = rows_lds + kChunkRows;
  UnitInfo u;
  if (!pick_unit<NFMAX <= 2>(chunks, n_chunks, H / 256 / G, G, u)) return;
  constexpr int GB = 8 * (FMT == 2 ? 8 : 12);
  const int wave = threadIdx.x >> 6, nkt = I / 64;
  // wave w copies rows 256 slice + 64 w .. + 63 of the expert
  const size_t row0 = (size_t)u.expert * H + 256 * u.slice0 + 64 * wave;
  const WeightTile wt = weight_tile<FMT>(down_codes, down_scales, row0, nkt);
  const strata_moe_expert_stats st = stats[u.expert];
  int tok = -1;
  if ((int)threadIdx.x < u.nfrag * 32) {  // one unit row per thread (at most 224)
    const int r = threadIdx.x, rr = r < u.nrows ? r : 0;
    const int slot = sorted_slot[u.row_start + rr];
    rows_lds[r] = u.row_start + rr;
    dst_lds[r] = slot;
    tok = slot / k;
  }
  __syncthreads();
  // a slice is 256 rows = 64 groups of 4
  const size_t wsl = (size_t)64 * nkt * GB, ssl = (size_t)64 * nkt * 8;
  // LDS weight tile w = rows 64 w .. 64 w + 63 of the slice
  const int ri = threadIdx.x & 31;
#define STRATA_DOWN_UNIT(NF)                                                                      \
  run_unit<FMT, NF, false, LDSB>(u, a16, I, I, rows_lds, dst_lds, wt, wsl, ssl, wave, wave, ri,    \
                                 32 + ri, st.shift_down, st.shift_down, xinfo, tok, st, expert_out, \
                                 H, 256, smem)
  if constexpr (NFMAX <= 2) {
    if (u.nfrag == 1) STRATA_DOWN_UNIT(1);
    else STRATA_DOWN_UNIT(2);
  } else {
    switch (u.nfrag) {
      case 1: STRATA_DOWN_UNIT(1); break;
      case 2: STRATA_DOWN_UNIT(2); break;
      case 3: STRATA_DOWN_UNIT(3); break;
      case 4: STRATA_DOWN_UNIT(4); break;
      case 5: STRATA_DOWN_UNIT(5); break;
      case 6: STRATA_DOWN_UNIT(6); break;
      default: STRATA_DOWN_UNIT(7); break;
    }
  }
#undef STRATA_DOWN_UNIT
}

// ---------------------------------------------------------------------------------------------
// Skinny grouped GEMMs: the small part's chunks of at most 32 rows (experts few tokens picked).
//
// With one fragment of rows every weight byte feeds one 32 x 32 tile of matrix work, so these
// units are bound by how fast they stream the expert's weights, not by the matrix cores.  Instead
// of the LDS stage ring of the kernels above (whose per-stage copies and barriers cap a thin
// unit's stream), each wave loads its own weights straight into registers, a ring of kSkDepth2
// (2-bit) or kSkDepth3 (3-bit) stages ahead of its matrix ops, with two 8-wave workgroups (16
// waves) per CU; the chunk's activation rows are staged once in LDS, in phases of the reduction
// where all of them do not fit.
//
// Operand layout.  A stage is 128 reduction indices, two 64-index tiles of the tiled layout.
// Lane (n, h) (n = lane % 32, h = lane / 32) loads weight row n's codes of tile 2j + h (both its
// blocks, 16 or 24 contiguous bytes) and their two scales, and feeds them as the B operand of
// steps 0..7 (steps 0-3 block 0, steps 4-7 block 1, 8 indices each in P8 order); the A operand of
// lane (m, h) holds the same 8 indices of activation row m, 16 contiguous bytes of the P8-ordered
// rows.  So every lane of a half-wave covers the same reduction indices, as the matrix op
// requires, and one wave load reads 8 row groups x 128 contiguous bytes (both tiles).

constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * 64;
// Dynamic LDS of a workgroup: the staged rows and, beside them, the output staging of 8 waves x 32
// rows x 80 bytes (two workgroups per CU with the 384 bytes of row tables).
constexpr int kSkLds = 81408;
constexpr int kSkOutRow = 80;  // bytes per row of a wave's output staging: 32 values + 16 pad
constexpr int kSkDepth2 = 3;   // stages of weights in flight per wave: 2-bit
constexpr int kSkDepth3 = 2;   // 3-bit (larger stages, more registers each)

template <int FMT>
struct SkStage {
  static constexpr int kW = FMT == 2 ? 4 : 6;  // code words of one row's two blocks
  uint32_t c0[kW], c1[kW];                     // the two streams' rows
  uint32_t s0, s1;                             // their two block scales (fp16, block 0 low)
};

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Default cache policy: a row group's scales of four consecutive stages share one 128-byte line
// (nontemporal loads measured 6 % slower: 252 against 237 us for the gate/up GEMM at T = 256).
template <int FMT>
STRATA_DEVICE void sk_load(SkStage<FMT>& r, const uint8_t* c0, const uint8_t* c1,
                           const uint16_t* s0, const uint16_t* s1) {
  if constexpr (FMT == 2) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(c0);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(c1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.c0[i] = a[i];
      r.c1[i] = b[i];
    }
  } else {  // 24 bytes at 8-byte alignment
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x2_t a = reinterpret_cast<const u32x2_t*>(c0)[i];
      const u32x2_t b = reinterpret_cast<const u32x2_t*>(c1)[i];
      r.c0[2 * i] = a[0];
      r.c0[2 * i + 1] = a[1];
      r.c1[2 * i] = b[0];
      r.c1[2 * i + 1] = b[1];
    }
  }
  r.s0 = *reinterpret_cast<const uint32_t*>(s0);
  r.s1 = *reinterpret_cast<const uint32_t*>(s1);
}

// One stage's 16 matrix ops; ap: this lane's 128 staged bytes of the stage (row m, tile 2j + h).
template <int FMT>
STRATA_DEVICE void sk_compute(f32x16_t& acc0, f32x16_t& acc1, const SkStage<FMT>& r,
                              const uint8_t* ap, int sh0, int sh1, const Q2Sel& ksel) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if constexpr (FMT == 2) {
      const Q2Tab t0 = q2_table((uint16_t)(r.s0 >> (16 * b)), sh0);
      const Q2Tab t1 = q2_table((uint16_t)(r.s1 >> (16 * b)), sh1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8_t a = *reinterpret_cast<const half8_t*>(ap + (4 * b + s) * 16);
        const half8_t w0 = q2_decode(r.c0[2 * b], r.c0[2 * b + 1], s, t0, ksel);
        const half8_t w1 = q2_decode(r.c1[2 * b], r.c1[2 * b + 1], s, t1, ksel);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w1, acc1, 0, 0, 0);
      }
    } else {
      const _Float16 e0 = __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)(r.s0 >> (16 * b))), sh0 + 2);
      const _Float16 e1 = __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)(r.s1 >> (16 * b))), sh1 + 2);
      const half2_t d40 = {e0, e0}, d41 = {e1, e1};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8_t a = *reinterpret_cast<const half8_t*>(ap + (4 * b + s) * 16);
        const half8_t w0 = q3_decode(r.c0[3 * b], r.c0[3 * b + 1], r.c0[3 * b + 2], s, d40);
        const half8_t w1 = q3_decode(r.c1[3 * b], r.c1[3 * b + 1], r.c1[3 * b + 2], s, d41);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w1, acc1, 0, 0, 0);
      }
    }
  }
}

// Stages the reduction indices [k0, k0 + klen) of the chunk's nr rows (source row row_src[m] of
// src, ld values long) into xs, rows rs bytes apart; four 16-byte pieces a thread per round.
STRATA_DEVICE void sk_stage_rows(uint8_t* xs, const uint16_t* __restrict__ src, int ld,
                                 const int* row_src, int nr, int k0, int klen, int rs) {
  const int per_row = klen >> 3, np = nr * per_row;
  for (int p0 = threadIdx.x; p0 < np; p0 += 4 * kSkThreads) {
    u32x4_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + i * kSkThreads;
      if (p < np) {
        const int m = p / per_row, c = p - m * per_row;
        v[i] = *reinterpret_cast<const u32x4_t*>(src + (size_t)row_src[m] * ld + k0 + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + i * kSkThreads;
      if (p < np) {
        const int m = p / per_row, c = p - m * per_row;
        *reinterpret_cast<u32x4_t*>(xs + m * rs + c * 16) = v[i];
      }
    }
  }
}

// UP: a16 rows of the chunk = SiLU(x W_g^T) * (x W_u^T) for 256 outputs of I per unit (wave w:
// outputs 32 w .. 32 w + 31 of the unit, gate rows as stream 0 and up rows as stream 1), NI = 1.
// !UP: expert_out rows = a W_d^T for 8 NI items of 64 rows of H per unit (wave w, item i: rows
// 64 (8 (unit part * NI + i) + w) .. + 63, its halves as the two streams).  upc: units per chunk.
// An item past the matrix's end repeats the last one and is not stored.
template <int FMT, bool UP, int P>
__global__ __launch_bounds__(kSkThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void ffn_skinny_kernel(
    const uint16_t* __restrict__ src, const XInfo* __restrict__ xinfo,
    const int* __restrict__ sorted_slot, int k, const Chunk* __restrict__ chunks,
    const int* __restrict__ n_chunks, const uint8_t* __restrict__ codes0,
    const uint8_t* __restrict__ codes1, const uint16_t* __restrict__ scales0,
    const uint16_t* __restrict__ scales1, const strata_moe_expert_stats* __restrict__ stats,
    int H, int I, int upc, int NI, uint16_t* __restrict__ out) {
  constexpr int CB = FMT == 2 ? 8 : 12;
  constexpr int GB = 8 * CB;  // code bytes of a 4-row group's 64-index tile
  __shared__ int row_src[kSkinnyRows], row_dst[kSkinnyRows], row_ex[kSkinnyRows];
  extern __shared__ __align__(16) uint8_t xs[];
  const int U = n_chunks[2] * upc;
  const int per = (U + 7) >> 3, bi = blockIdx.x >> 3;
  if (bi >= per) return;
  const int unit = (blockIdx.x & 7) * per + bi;  // consecutive units on one XCD
  if (unit >= U) return;
  const Chunk ch = chunks[unit / upc];
  const int part = unit % upc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, h = lane >> 5;
  const int K = UP ? H : I, nkt = K / 64, NS = K / 128, nr = ch.nrows;
  const strata_moe_expert_stats st = stats[ch.expert];
  // phases: the longest run of whole stages whose nr rows fit, spread evenly over the phases
  const int kfit = (kSkLds / (2 * nr) - 8) & ~127;
  const int nph = (K + kfit - 1) / kfit, sp = (NS + nph - 1) / nph;  // stages per phase
  const int rs = (sp * 128 + 8) * 2;                                  // bytes per staged row
  // output staging beside the staged rows when the items share them (NI > 1: one phase, and the
  // launch checks that 32 rows and the 8 regions fit)
  uint8_t* const ep_tail = xs + ((nr * rs + 15) & ~15);
  const int NT = NI * NS;
  const int sh0 = UP ? st.shift_gate : st.shift_down, sh1 = UP ? st.shift_up : st.shift_down;
  const int R = UP ? I : H;  // rows of one expert's matrix
  // Loads address the expert's tiles from a uniform base plus this lane's fixed 32-bit offset
  // (the item's rows, its tile h); a stage adds 2 tiles to the uniform part.
  const size_t eg = (size_t)ch.expert * (R / 4) * nkt;  // the expert's first row group x tiles
  const uint8_t* const cb0 = codes0 + eg * GB;
  const uint8_t* const cb1 = codes1 + eg * GB;
  const uint16_t* const sb0 = scales0 + eg * 8;
  const uint16_t* const sb1 = scales1 + eg * 8;
  // first output of item it (past the matrix: not stored), and this lane's offsets for it
  auto item_first = [&](int it) {
    return UP ? part * 256 + wave * 32 : 64 * ((part * NI + it) * kSkWaves + wave);
  };
  auto lane_offsets = [&](int it, uint32_t& oc0, uint32_t& oc1, uint32_t& os0, uint32_t& os1) {
    const int rr = min(item_first(it), R - (UP ? 32 : 64)) + n;  // stream 0's row
    const uint32_t t = (uint32_t)((rr >> 2) * nkt + h);
    oc0 = t * GB + (rr & 3) * 2 * CB;
    os0 = t * 8 + (rr & 3) * 2;
    oc1 = UP ? oc0 : oc0 + 8 * nkt * GB;  // down: stream 1 is 32 rows (8 groups) further
    os1 = UP ? os0 : os0 + 8 * nkt * 8;
  };
  int lit = 0, ljs = 0;  // load cursor: item, stage
  uint32_t oc0, oc1, os0, os1;
  lane_offsets(0, oc0, oc1, os0, os1);
  // Every stage slot issues the same loads unconditionally (the compiler's counter waits then see
  // the same loads in flight on every path and wait for exactly one stage): past the last stage
  // they read the first 128 bytes of the (cache-resident) activation rows instead (at least 256
  // bytes exist), selected branch-free.
  const uint8_t* const dsrc = reinterpret_cast<const uint8_t*>(src);
  const uint32_t doff = (lane & 7) * 16;
  auto load_next = [&](SkStage<FMT>& r) {
    const bool live = lit < NI;
    const size_t sc = (size_t)ljs * 2 * GB, ss = (size_t)ljs * 16;
    const uint8_t* p0 = live ? cb0 + sc : dsrc;
    const uint8_t* p1 = live ? cb1 + sc : dsrc;
    const uint8_t* q0 = live ? reinterpret_cast<const uint8_t*>(sb0 + ss) : dsrc;
    const uint8_t* q1 = live ? reinterpret_cast<const uint8_t*>(sb1 + ss) : dsrc;
    sk_load<FMT>(r, p0 + (live ? oc0 : doff), p1 + (live ? oc1 : doff),
                 reinterpret_cast<const uint16_t*>(q0 + (live ? 2 * os0 : doff)),
                 reinterpret_cast<const uint16_t*>(q1 + (live ? 2 * os1 : doff)));
    if (live && ++ljs == NS) {
      ljs = 0;
      if (++lit < NI) lane_offsets(lit, oc0, oc1, os0, os1);
    }
  };
  // the first stages' weights first, so that their latency overlaps the row tables' dependent loads
  SkStage<FMT> ring[P];
#pragma unroll
  for (int i = 0; i < P; ++i) load_next(ring[i]);
  if (tid < nr) {
    const int slot = sorted_slot[ch.row_start + tid], tok = slot / k;
    row_src[tid] = UP ? tok : ch.row_start + tid;
    row_dst[tid] = UP ? ch.row_start + tid : slot;
    row_ex[tid] = row_exponent<UP>(xinfo[tok], st);
  }
  __syncthreads();  // row tables
  sk_stage_rows(xs, src, K, row_src, nr, 0, min(K, sp * 128), rs);
  __syncthreads();  // staged rows
  const Q2Sel ksel = q2_sel();
  // rows past the chunk read row nr - 1 (their results are not stored)
  const uint8_t* arow = xs + min(n, nr - 1) * rs + h * 128;
  f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
  int it = 0, js = 0, jp = 0;  // compute cursor: item, stage, stage within the staged phase
  // one stage from ring slot r: the next phase first if due, the item's outputs after its last
  // stage
  auto stage = [&](SkStage<FMT>& r) {
    if (jp == sp) {  // the next phase (uniform across the workgroup)
      jp = 0;
      __syncthreads();
      sk_stage_rows(xs, src, K, row_src, nr, js * 128, min(K - js * 128, sp * 128), rs);
      __syncthreads();
    }
    sk_compute<FMT>(acc0, acc1, r, arow + jp * 256, sh0, sh1, ksel);
    ++jp;
    if (++js == NS) {  // the item's outputs
      const int first = item_first(it);
      // Through this wave's LDS region, so that every store is a 16-byte piece (2-byte stores
      // from 32 lanes cost a write request each).  Items that share the staged rows (NI > 1)
      // use the space beside them; a single item's region overlays the rows once every wave is
      // done with them.
      uint8_t* reg;
      if (NI > 1) {
        reg = ep_tail + wave * nr * kSkOutRow;
      } else {
        __syncthreads();
        reg = xs + wave * nr * kSkOutRow;
      }
      if (first < R) {
        // register q of this lane holds row 8 (q >> 2) + 4 h + (q & 3): one base per lane and
        // constant offsets (the base is opaque so that nothing of it is held across the loop)
        int lim = nr - 4 * h;  // rows 4 h + d exist for d < lim
        uint32_t lo = (uint32_t)(4 * h * kSkOutRow) + 2u * (UP ? (n & ~7) + p8inv(n & 7) : n);
        asm volatile("" : "+v"(lo), "+v"(lim));
        uint8_t* const lb = reg + lo;
        const int* const exr = row_ex + 4 * h;
#pragma unroll
        for (int pass = 0; pass < (UP ? 1 : 2); ++pass) {  // down: the two 32-row halves
#pragma unroll
          for (int q = 0; q < 16; q += 2) {  // rows d and d + 1 (q and q + 1 share q >> 2)
            const int d = 8 * (q >> 2) + (q & 3);
            uint16_t v0, v1;
            if constexpr (UP) {
              const int e0 = exr[d], e1 = exr[d + 1];
              v0 = __builtin_bit_cast(uint16_t, silu_mul_scaled(acc0[q], acc1[q], (int)(int16_t)(e0 & 0xFFFF), e0 >> 16));
              v1 = __builtin_bit_cast(uint16_t, silu_mul_scaled(acc0[q + 1], acc1[q + 1], (int)(int16_t)(e1 & 0xFFFF), e1 >> 16));
            } else {
              const uint32_t b = bf16_pair_rne(__builtin_ldexpf(pass ? acc1[q] : acc0[q], exr[d]),
                                               __builtin_ldexpf(pass ? acc1[q + 1] : acc0[q + 1], exr[d + 1]));
              v0 = (uint16_t)b;
              v1 = (uint16_t)(b >> 16);
            }
            if (d < lim) *reinterpret_cast<uint16_t*>(lb + d * kSkOutRow) = v0;
            if (d + 1 < lim) *reinterpret_cast<uint16_t*>(lb + (d + 1) * kSkOutRow) = v1;
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's values are in place
          for (int pc = lane; pc < 4 * nr; pc += 64) {  // 4 pieces of 8 values per row
            const int m = pc >> 2, c = pc & 3;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(reg + m * kSkOutRow + c * 16);
            if constexpr (UP) {
              *reinterpret_cast<u32x4_t*>(out + (size_t)row_dst[m] * I + first + 8 * c) = v;
            } else {  // expert outputs: read once, by the combine
              __builtin_nontemporal_store(
                  v, reinterpret_cast<u32x4_t*>(out + (size_t)row_dst[m] * H + first + 32 * pass + 8 * c));
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next pass writes
        }
      }
      acc0 = f32x16_t{};
      acc1 = f32x16_t{};
      js = 0;
      ++it;
      jp = sp < NS ? sp : 0;  // several phases: the next item restages the first
    }
  };
  // whole groups of P stages, the last one computing only the stages that exist; every slot is
  // refilled (past the end from the activation line), so that no path holds fewer loads in flight
  // and no separate tail keeps values alive across the loop
  for (int j0 = 0; j0 < NT; j0 += P) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (j0 + i < NT) stage(ring[i]);
      load_next(ring[i]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// x bf16 -> fp16 in P8 order, scaled per token: one wave per row.  The row's largest |x| (bf16
// magnitudes order as their bit patterns) fixes sx with max |x| 2^sx in [2^14, 2^15); each value
// is then x 2^sx, exact in fp16 (8 significant bits, no overflow; values below 2^-17 of the
// scaled maximum round into fp16's subnormals), and n2 = sum of the squares of the fp16 values.

constexpr int kXRowsPerBlock = 4;
constexpr int kXRegPieces = 8;  // 16-byte pieces a lane keeps in registers (rows up to 4096)

STRATA_DEVICE uint32_t bf16_pair_max_mag(uint32_t v, uint32_t m) {
  return max(m, max(v & 0x7FFFu, (v >> 16) & 0x7FFFu));
}

STRATA_DEVICE u32x4_t x_piece_to_f16(const u32x4_t v, int sx, float& n2) {
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
    const _Float16 lo = (_Float16)__builtin_ldexpf(bf16_to_f32(in[P8[2 * m]]), sx);
    const _Float16 hi = (_Float16)__builtin_ldexpf(bf16_to_f32(in[P8[2 * m + 1]]), sx);
    const float flo = (float)lo, fhi = (float)hi;
    n2 = __builtin_fmaf(flo, flo, n2);
    n2 = __builtin_fmaf(fhi, fhi, n2);
    o[m] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return o;
}

// Row t (this wave).
STRATA_DEVICE void x_to_f16_row(const uint16_t* __restrict__ x, int t, int H, uint16_t* __restrict__ x16,
                                XInfo* __restrict__ xinfo) {
  const int lane = threadIdx.x & 63;
  const int n8 = H / 8;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)t * H);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(x16 + (size_t)t * H);
  u32x4_t v[kXRegPieces];
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < kXRegPieces; ++j) {
    const int i = lane + 64 * j;
    v[j] = i < n8 ? __builtin_nontemporal_load(src + i) : u32x4_t{0, 0, 0, 0};  // x is read once
#pragma unroll
    for (int m = 0; m < 4; ++m) mx = bf16_pair_max_mag(v[j][m], mx);
  }
  for (int i = lane + 64 * kXRegPieces; i < n8; i += 64) {  // rows longer than 4096
    const u32x4_t w = src[i];
#pragma unroll
    for (int m = 0; m < 4; ++m) mx = bf16_pair_max_mag(w[m], mx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  // max |x| in [2^(e-1), 2^e): sx = 15 - e
  const int sx = mx ? 15 - __builtin_amdgcn_frexp_expf(bf16_to_f32((uint16_t)mx)) : 0;
  float n2 = 0.0f;
#pragma unroll
  for (int j = 0; j < kXRegPieces; ++j) {
    const int i = lane + 64 * j;
    if (i < n8) dst[i] = x_piece_to_f16(v[j], sx, n2);
  }
  for (int i = lane + 64 * kXRegPieces; i < n8; i += 64) dst[i] = x_piece_to_f16(src[i], sx, n2);
  n2 = wave_sum(n2);
  if (lane == 0) xinfo[t] = XInfo{sx, n2};
}

__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                       uint16_t* __restrict__ x16,
                                                       XInfo* __restrict__ xinfo) {
  const int t = blockIdx.x * kXRowsPerBlock + (threadIdx.x >> 6);
  if (t < T) x_to_f16_row(x, t, H, x16, xinfo);
}

// The layer call's first launch: the router's top-k (workgroups [0, nroute), one wave per token,
// the selection of route_kernel) and the conversion of x above (the other workgroups, one wave per
// row).  The two steps are independent, and each would otherwise pay a launch of its own.
template <int NPL>
__global__ __launch_bounds__(64 * kXRowsPerBlock) void route_x16_kernel(
    const float* __restrict__ logits, int T, int E, int k, int* __restrict__ ids,
    float* __restrict__ w, int nroute, const uint16_t* __restrict__ x, int H,
    uint16_t* __restrict__ x16, XInfo* __restrict__ xinfo) {
  __shared__ __align__(16) uint64_t sel[kXRowsPerBlock][80];
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < nroute) {
    const int t = blockIdx.x * kXRowsPerBlock + wave;
    if (t >= T) return;
    TokenKeys<NPL> tk;
    load_token_logits<NPL>(logits + (size_t)t * E, E, tk);
    select_token_wave<NPL>(tk, E, k, ids + (size_t)t * k, w + (size_t)t * k, sel[wave]);
    return;
  }
  const int t = (blockIdx.x - nroute) * kXRowsPerBlock + wave;
  if (t < T) x_to_f16_row(x, t, H, x16, xinfo);
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t][h] (+)= sum_j w[t][j] * out[t*k + j][h], j ascending (one thread per 8 h).

constexpr int kCombineMaxK = 16;  // rows requested together (the largest k the router takes)

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
  // all k rows requested before the first is used (k <= 16)
  u32x4_t v[kCombineMaxK];
  float wj[kCombineMaxK];
#pragma unroll
  for (int j = 0; j < kCombineMaxK; ++j) {
    if (j < k) {
      wj[j] = w[(size_t)t * k + j];
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(out + ((size_t)t * k + j) * H + c * 8));
    }
  }
#pragma unroll
  for (int j = 0; j < kCombineMaxK; ++j) {
    if (j < k) {
      const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        s[2 * m] = __builtin_fmaf(wj[j], __uint_as_float(q[m] << 16), s[2 * m]);
        s[2 * m + 1] = __builtin_fmaf(wj[j], __uint_as_float(q[m] & 0xFFFF0000u), s[2 * m + 1]);
      }
    }
  }
  for (int j = kCombineMaxK; j < k; ++j) {  // k > 16: only through strata_moe_combine
    const float wr = w[(size_t)t * k + j];
    const u32x4_t vr = *reinterpret_cast<const u32x4_t*>(out + ((size_t)t * k + j) * H + c * 8);
    const uint32_t q[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[2 * m] = __builtin_fmaf(wr, __uint_as_float(q[m] << 16), s[2 * m]);
      s[2 * m + 1] = __builtin_fmaf(wr, __uint_as_float(q[m] & 0xFFFF0000u), s[2 * m + 1]);
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

// Slices per unit: the largest divisor of n_slices not above gmax that still leaves about two
// units per CU for the fewest chunks S slots can make.  More slices per unit pay the unit's fixed
// costs (launch, row tables, pipeline fill) once for several slices; fewer keep enough units to
// fill and balance the CUs (a skewed routing concentrates the slots in few chunks).
static int slices_per_unit(int n_slices, int gmax, int64_t S, int chunk_rows) {
  const int64_t min_chunks = (S + chunk_rows - 1) / chunk_rows;
  for (int g = gmax; g > 1; --g)
    if (n_slices % g == 0 && min_chunks * (n_slices / g) >= 2 * 256) return g;
  return 1;
}

// The GEMM kernels use more than 64 KB of dynamic LDS; allow it once per process.
static void allow_big_lds() {
  static std::once_flag once;
  std::call_once(once, [] {
    const void* big[4] = {reinterpret_cast<const void*>(ffn_up_kernel<2, 7>),
                          reinterpret_cast<const void*>(ffn_up_kernel<3, 7>),
                          reinterpret_cast<const void*>(ffn_down_kernel<2, 7>),
                          reinterpret_cast<const void*>(ffn_down_kernel<3, 7>)};
    const void* small[4] = {reinterpret_cast<const void*>(ffn_up_kernel<2, 2>),
                            reinterpret_cast<const void*>(ffn_up_kernel<3, 2>),
                            reinterpret_cast<const void*>(ffn_down_kernel<2, 2>),
                            reinterpret_cast<const void*>(ffn_down_kernel<3, 2>)};
    for (const void* k : big)
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
    for (const void* k : small)
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLdsSmall);
    const void* skinny[4] = {reinterpret_cast<const void*>(ffn_skinny_kernel<2, true, kSkDepth2>),
                             reinterpret_cast<const void*>(ffn_skinny_kernel<3, true, kSkDepth3>),
                             reinterpret_cast<const void*>(ffn_skinny_kernel<2, false, kSkDepth2>),
                             reinterpret_cast<const void*>(ffn_skinny_kernel<3, false, kSkDepth3>)};
    for (const void* k : skinny)
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkLds);
  });
}

hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, XInfo* xinfo,
                           hipStream_t s) {
  const unsigned grid = (unsigned)((T + kXRowsPerBlock - 1) / kXRowsPerBlock);
  x_to_f16_kernel<<<grid, 256, 0, s>>>(x, T, H, x16, xinfo);
  return hipGetLastError();
}

hipError_t launch_route_x16(const float* logits, int T, int E, int k, int* ids, float* w,
                            const uint16_t* x, int H, uint16_t* x16, XInfo* xinfo, hipStream_t s) {
  const int n = (T + kXRowsPerBlock - 1) / kXRowsPerBlock;  // workgroups of each half
  const dim3 grid(2 * n), block(64 * kXRowsPerBlock);
  if (E <= 64) route_x16_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, n, x, H, x16, xinfo);
  else if (E <= 128) route_x16_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, n, x, H, x16, xinfo);
  else if (E <= 256) route_x16_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, n, x, H, x16, xinfo);
  else if (E <= 512) route_x16_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, n, x, H, x16, xinfo);
  else route_x16_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, n, x, H, x16, xinfo);
  return hipGetLastError();
}

hipError_t launch_ffn_up(int fmt, const uint16_t* x16, const XInfo* xinfo, const int* sorted_slot,
                         int k, int64_t S, const Chunk* chunks, const int* n_chunks, int max_small,
                         int max_large, const void* gate_codes, const void* up_codes,
                         const uint16_t* gate_scales, const uint16_t* up_scales,
                         const strata_moe_expert_stats* stats, int E, int H, int I, uint16_t* a16,
                         hipStream_t s) {
  (void)E;
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  allow_big_lds();
#define STRATA_LAUNCH_UP(F, NFM, LDSB, CH, NCH, G, GRID)                                          \
  ffn_up_kernel<F, NFM><<<GRID, kGemmThreads, LDSB, s>>>(x16, xinfo, sorted_slot, k, CH, NCH, gc, uc, \
                                                         gate_scales, up_scales, stats, H, I, G, a16)
  if (max_small > 0) {  // the small part's skinny chunks: 256 outputs per unit
    const int upc = (I + 255) / 256;
    const int grid = grid_for_units((int64_t)max_small * upc);
    if (fmt == 2)
      ffn_skinny_kernel<2, true, kSkDepth2><<<grid, kSkThreads, kSkLds, s>>>(
          x16, xinfo, sorted_slot, k, chunks, n_chunks, gc, uc, gate_scales, up_scales, stats, H, I,
          upc, 1, a16);
    else
      ffn_skinny_kernel<3, true, kSkDepth3><<<grid, kSkThreads, kSkLds, s>>>(
          x16, xinfo, sorted_slot, k, chunks, n_chunks, gc, uc, gate_scales, up_scales, stats, H, I,
          upc, 1, a16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the rest of the small part has chunks of more than kSkinnyRows rows
  const int64_t max_rest = max_rest_chunks(S, max_small);
  if (max_rest > 0) {  // the rest of the small part: one slice per unit
    const int grid = grid_for_units(max_rest * (I / 128));
    if (fmt == 2) STRATA_LAUNCH_UP(2, 2, kGemmLdsSmall, chunks, n_chunks, 1, grid);
    else STRATA_LAUNCH_UP(3, 2, kGemmLdsSmall, chunks, n_chunks, 1, grid);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = slices_per_unit(I / 128, 1, S, kChunkRows);
  const int grid = grid_for_units((int64_t)max_large * (I / 128 / G));
  if (fmt == 2) STRATA_LAUNCH_UP(2, 7, kGemmLds, chunks + max_small, n_chunks + 1, G, grid);
  else STRATA_LAUNCH_UP(3, 7, kGemmLds, chunks + max_small, n_chunks + 1, G, grid);
#undef STRATA_LAUNCH_UP
  return hipGetLastError();
}

hipError_t launch_ffn_down(int fmt, const uint16_t* a16, const XInfo* xinfo,
                           const int* sorted_slot, int k, int64_t S, const Chunk* chunks,
                           const int* n_chunks, int max_small, int max_large,
                           const void* down_codes, const uint16_t* down_scales,
                           const strata_moe_expert_stats* stats, int E, int H, int I,
                           uint16_t* expert_out, hipStream_t s) {
  (void)E;
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  allow_big_lds();
#define STRATA_LAUNCH_DOWN(F, NFM, LDSB, CH, NCH, G, GRID)                                        \
  ffn_down_kernel<F, NFM><<<GRID, kGemmThreads, LDSB, s>>>(a16, xinfo, sorted_slot, k, CH, NCH, dc, \
                                                           down_scales, stats, H, I, G, expert_out)
  if (max_small > 0) {  // the small part's skinny chunks
    // items of 64 rows of H; about 16 per wave (two units per chunk) while one phase holds a's
    // rows and the output staging beside them (the items of a wave then share the staged rows),
    // else one
    const int items = H / 64;
    const bool share = kSkinnyRows * (I + 8) * 2 + 16 + kSkWaves * kSkinnyRows * kSkOutRow <= kSkLds;
    const int NI = share ? (items + 15) / 16 : 1;
    const int upc = (items + kSkWaves * NI - 1) / (kSkWaves * NI);
    const int grid = grid_for_units((int64_t)max_small * upc);
    if (fmt == 2)
      ffn_skinny_kernel<2, false, kSkDepth2><<<grid, kSkThreads, kSkLds, s>>>(
          a16, xinfo, sorted_slot, k, chunks, n_chunks, dc, dc, down_scales, down_scales, stats, H,
          I, upc, NI, expert_out);
    else
      ffn_skinny_kernel<3, false, kSkDepth3><<<grid, kSkThreads, kSkLds, s>>>(
          a16, xinfo, sorted_slot, k, chunks, n_chunks, dc, dc, down_scales, down_scales, stats, H,
          I, upc, NI, expert_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t max_rest = max_rest_chunks(S, max_small);
  if (max_rest > 0) {  // the rest of the small part: two slices per unit (24 stages: K = I is short)
    const int Gs = (H / 256) % 2 == 0 ? 2 : 1;
    const int grid = grid_for_units(max_rest * (H / 256 / Gs));
    if (fmt == 2) STRATA_LAUNCH_DOWN(2, 2, kGemmLdsSmall, chunks, n_chunks, Gs, grid);
    else STRATA_LAUNCH_DOWN(3, 2, kGemmLdsSmall, chunks, n_chunks, Gs, grid);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = slices_per_unit(H / 256, 2, S, kChunkRows);
  const int grid = grid_for_units((int64_t)max_large * (H / 256 / G));
  if (fmt == 2) STRATA_LAUNCH_DOWN(2, 7, kGemmLds, chunks + max_small, n_chunks + 1, G, grid);
  else STRATA_LAUNCH_DOWN(3, 7, kGemmLds, chunks + max_small, n_chunks + 1, G, grid);
#undef STRATA_LAUNCH_DOWN
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
