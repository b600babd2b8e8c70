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
constexpr int kGemmLds = 160 * 1024;              // the whole LDS of a CU
constexpr int kRowsBytes = 2 * kChunkRows * 4;    // a unit's source and destination rows
// Output staging: two 32-row buffers (one fragment each) with padded rows.
constexpr int kUpOutRow = 128 + 8;                // halfs per row: 128 outputs
constexpr int kDownOutRow = 256 + 8;              // halfs per row: 256 outputs
constexpr int kUpEpiBytes = 2 * 32 * kUpOutRow * 2;
constexpr int kDownEpiBytes = 2 * 32 * kDownOutRow * 2;

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
// a contiguous range, so the slice groups of one chunk run side by side on one L2.
STRATA_DEVICE bool pick_unit(const Chunk* chunks, const int* n_chunks, int n_groups, int G,
                             UnitInfo& u) {
  const int U = *n_chunks * n_groups;
  const int per = (U + 7) >> 3;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  if (i >= per) return false;
  const int unit = xcd * per + i;
  if (unit >= U) return false;
  const Chunk ch = chunks[unit / n_groups];
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
                                      int ri0, int ri1, int hh) {
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
    sw.t0 = q2_table(d0);
    sw.t1 = q2_table(d1);
  } else {
    const _Float16 e0 = __builtin_bit_cast(_Float16, d0) * (_Float16)4.0f;  // exact
    const _Float16 e1 = __builtin_bit_cast(_Float16, d1) * (_Float16)4.0f;
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

STRATA_DEVICE float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Writes one slice's outputs, fragment by fragment, through two LDS staging buffers, with 16-byte
// stores.  Up: out = A (fp16, [rows][I], columns in P8 order within groups of 8), 128 outputs per
// slice, lane c < 16 of a tile holding the gate and lane c + 16 the up value of output 16 w + c ...
// (acc0 = gate, acc1 = up columns); down: out = expert outputs (bf16, [slots][H]), 256 per slice.
// dst_lds[r]: the destination row of unit row r (rows past the chunk repeat row 0, whose values
// they equal, so every lane stores).  Each wave issues kStores stores per fragment.
template <int NF, bool UP>
struct Epilogue {
  static constexpr int kRow = UP ? kUpOutRow : kDownOutRow;        // halfs per staged row
  static constexpr int kPieces = UP ? 16 : 32;                     // 16-byte pieces per row
  static constexpr int kStores = 32 * kPieces / kGemmThreads;      // per thread per fragment
  static constexpr int kBuf = 32 * kRow;                           // halfs per staging buffer
};

template <int NF, bool UP>
STRATA_DEVICE void write_slice(f32x16_t (&acc0)[NF], f32x16_t (&acc1)[NF], uint16_t* epi,
                               const int* dst_lds, uint16_t* __restrict__ out, int out_ld, int col0) {
  using EP = Epilogue<NF, UP>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  // this lane's first staged element (tile row 4 hh, its column); register r of a tile adds
  // rows 8 (r >> 2) + (r & 3), a constant offset
  const int lcol = UP ? wave * 32 + (nl & ~7) + p8inv(nl & 7) : wave * 64 + nl;
  uint16_t* const e0 = epi + 4 * hh * EP::kRow + lcol;
  // (opaque to the optimizer, so that the store addresses are not computed once for every slice
  // and held in registers across the main loop)
  asm volatile("" : "+s"(out_ld));
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    // One fragment at a time: the empty asm re-defines this fragment's sums in the accumulation
    // registers here, so their copies into VGPRs cannot be hoisted above it (all fragments'
    // copies at once would need 32 NF VGPRs).
    asm volatile("" : "+a"(acc0[f]), "+a"(acc1[f]));
    uint16_t* eb = e0 + (f & 1) * EP::kBuf;
    if constexpr (UP) {
      // acc0 columns: gate of outputs w*32 + n; acc1: up of the same outputs
#pragma unroll
      for (int r = 0; r < 16; ++r)
        eb[(8 * (r >> 2) + (r & 3)) * EP::kRow] =
            __builtin_bit_cast(uint16_t, f32_to_f16_sat(silu_mul(acc0[f][r], acc1[f][r])));
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        eb[(8 * (r >> 2) + (r & 3)) * EP::kRow] = f32_to_bf16(acc0[f][r]);
        eb[(8 * (r >> 2) + (r & 3)) * EP::kRow + 32] = f32_to_bf16(acc1[f][r]);
      }
    }
    // the buffer is complete for every wave; (the other buffer's previous reads finished before
    // each wave's own barrier here, so the next fragment may overwrite it)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    const uint16_t* rb = epi + (f & 1) * EP::kBuf;
#pragma unroll
    for (int i = 0; i < EP::kStores; ++i) {
      const int p = threadIdx.x + i * kGemmThreads;
      const int r = p / EP::kPieces, c = p % EP::kPieces;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(rb + r * EP::kRow + c * 8);
      *reinterpret_cast<u32x4_t*>(out + (size_t)dst_lds[f * 32 + r] * out_ld + col0 + c * 8) = v;
    }
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
                               int ri1, const Q2Sel& ksel) {
  const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
  load_stage_weights<FMT, NF>(ss.sw, st, ti0, ti1, ri0, ri1, hh);
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
// (ti, ri): this lane's B rows in the LDS weight tiles; out/out_ld/ocols: destination and the
// columns per slice.
template <int FMT, int NF, bool UP>
STRATA_DEVICE void run_unit(const UnitInfo& u, const uint16_t* __restrict__ src, int ld, int K,
                            const int* rows_lds, const int* dst_lds, const WeightTile& wt,
                            size_t wslice, size_t sslice, int ti0, int ti1, int ri0, int ri1,
                            uint16_t* __restrict__ out, int out_ld, int ocols, uint8_t* lds) {
  constexpr int kEpi = UP ? kUpEpiBytes : kDownEpiBytes;
  using P = Pipe<FMT, NF, kGemmLds - kRowsBytes - kEpi>;
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
  CopyCursor cc{0, 0, NT, NKs, 0, 0, wslice, sslice};
#pragma unroll
  for (int j = 0; j < P::kPD; ++j)
    if (j < NT) {
      issue_copies<FMT, NF>(lds + j * P::kStage, src, xoff, wt, cc.ks, cc.woff, cc.soff, 0, P::kPer);
      cursor_advance<FMT>(cc);
    }
  stage_barrier<P::kPer * (P::kPD - 1)>(ops_after<P::kPer, P::kPD>(0, -1, NT, NKs, kSt));
  const Q2Sel ksel = q2_sel();
  StageState<FMT, NF> ss;
  stage_setup<FMT, NF>(ss, lds, ti0, ti1, ri0, ri1, ksel);
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
      stage_setup<FMT, NF>(ss, lds + nb * P::kStage, ti0, ti1, ri0, ri1, ksel);
      mfma_step<NF>(acc0, acc1, ss.a[1], ss.b[1], kPre, NF);
      __builtin_amdgcn_sched_barrier(0);
      rb = nb;
    }
    // (the staging area is separate from the stage ring, which the next slice's copies fill)
    write_slice<NF, UP>(acc0, acc1, epi, dst_lds, out, out_ld, (u.slice0 + sl) * ocols);
    last_end = j - 1;
  }
}

// ---------------------------------------------------------------------------------------------
// Up projection: A[p][n] = SiLU(x_t . W_g[n]) * (x_t . W_u[n]) for the chunk's rows p.
// Slice = 128 outputs; wave w owns outputs slice*128 + w*32 + (lane % 32), gate and up.

template <int FMT>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_up_kernel(
    const uint16_t* __restrict__ x16, const int* __restrict__ sorted_slot, int k,
    const Chunk* __restrict__ chunks, const int* __restrict__ n_chunks,
    const uint8_t* __restrict__ gate_codes, const uint8_t* __restrict__ up_codes,
    const uint16_t* __restrict__ gate_scales, const uint16_t* __restrict__ up_scales, int H, int I,
    int G, uint16_t* __restrict__ a16) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* rows_lds = reinterpret_cast<int*>(smem + kGemmLds - kRowsBytes);
  int* dst_lds = rows_lds + kChunkRows;
  UnitInfo u;
  if (!pick_unit(chunks, n_chunks, I / 128 / G, G, u)) return;
  constexpr int GB = 8 * (FMT == 2 ? 8 : 12);
  const int wave = threadIdx.x >> 6, nkt = H / 64;
  // wave w copies gate (w < 2) or up rows 128 slice + 64 (w & 1) .. + 63 of the expert
  const size_t row0 = (size_t)u.expert * I + 128 * u.slice0 + 64 * (wave & 1);
  const WeightTile wt = weight_tile<FMT>(wave < 2 ? gate_codes : up_codes,
                                         wave < 2 ? gate_scales : up_scales, row0, nkt);
  for (int r = threadIdx.x; r < u.nfrag * 32; r += kGemmThreads) {
    const int rr = r < u.nrows ? r : 0;
    rows_lds[r] = sorted_slot[u.row_start + rr] / k;
    dst_lds[r] = u.row_start + rr;
  }
  __syncthreads();
  // a slice is 128 gate (and up) rows = 32 groups of 4
  const size_t wsl = (size_t)32 * nkt * GB, ssl = (size_t)32 * nkt * 8;
  // LDS weight tiles 0, 1 = gate rows 0-63, 64-127 of the slice; 2, 3 = the same up rows
  const int ri = (wave & 1) * 32 + (threadIdx.x & 31);
#define STRATA_UP_UNIT(NF)                                                                        \
  run_unit<FMT, NF, true>(u, x16, H, H, rows_lds, dst_lds, wt, wsl, ssl, wave >> 1, 2 + (wave >> 1), \
                          ri, ri, a16, I, 128, smem)
  switch (u.nfrag) {
    case 1: STRATA_UP_UNIT(1); break;
    case 2: STRATA_UP_UNIT(2); break;
    case 3: STRATA_UP_UNIT(3); break;
    case 4: STRATA_UP_UNIT(4); break;
    case 5: STRATA_UP_UNIT(5); break;
    case 6: STRATA_UP_UNIT(6); break;
    default: STRATA_UP_UNIT(7); break;
  }
#undef STRATA_UP_UNIT
}

// ---------------------------------------------------------------------------------------------
// Down projection: out[slot(p)][h] = A[p] . W_d[h] for the chunk's rows p, written as bf16 in
// slot order.  Slice = 256 outputs; wave w owns h = slice*256 + w*64 + nf*32 + (lane % 32).

template <int FMT>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_down_kernel(
    const uint16_t* __restrict__ a16, const int* __restrict__ sorted_slot,
    const Chunk* __restrict__ chunks, const int* __restrict__ n_chunks,
    const uint8_t* __restrict__ down_codes, const uint16_t* __restrict__ down_scales, int H, int I,
    int G, uint16_t* __restrict__ expert_out) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* rows_lds = reinterpret_cast<int*>(smem + kGemmLds - kRowsBytes);
  int* dst_lds = rows_lds + kChunkRows;
  UnitInfo u;
  if (!pick_unit(chunks, n_chunks, H / 256 / G, G, u)) return;
  constexpr int GB = 8 * (FMT == 2 ? 8 : 12);
  const int wave = threadIdx.x >> 6, nkt = I / 64;
  // wave w copies rows 256 slice + 64 w .. + 63 of the expert
  const size_t row0 = (size_t)u.expert * H + 256 * u.slice0 + 64 * wave;
  const WeightTile wt = weight_tile<FMT>(down_codes, down_scales, row0, nkt);
  for (int r = threadIdx.x; r < u.nfrag * 32; r += kGemmThreads) {
    const int rr = r < u.nrows ? r : 0;
    rows_lds[r] = u.row_start + rr;
    dst_lds[r] = sorted_slot[u.row_start + rr];
  }
  __syncthreads();
  // a slice is 256 rows = 64 groups of 4
  const size_t wsl = (size_t)64 * nkt * GB, ssl = (size_t)64 * nkt * 8;
  // LDS weight tile w = rows 64 w .. 64 w + 63 of the slice
  const int ri = threadIdx.x & 31;
#define STRATA_DOWN_UNIT(NF)                                                                      \
  run_unit<FMT, NF, false>(u, a16, I, I, rows_lds, dst_lds, wt, wsl, ssl, wave, wave, ri, 32 + ri, \
                           expert_out, H, 256, smem)
  switch (u.nfrag) {
    case 1: STRATA_DOWN_UNIT(1); break;
    case 2: STRATA_DOWN_UNIT(2); break;
    case 3: STRATA_DOWN_UNIT(3); break;
    case 4: STRATA_DOWN_UNIT(4); break;
    case 5: STRATA_DOWN_UNIT(5); break;
    case 6: STRATA_DOWN_UNIT(6); break;
    default: STRATA_DOWN_UNIT(7); break;
  }
#undef STRATA_DOWN_UNIT
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
      v[j] = *reinterpret_cast<const u32x4_t*>(out + ((size_t)t * k + j) * H + c * 8);
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
static int slices_per_unit(int n_slices, int gmax, int64_t S) {
  const int64_t min_chunks = (S + kChunkRows - 1) / kChunkRows;
  for (int g = gmax; g > 1; --g)
    if (n_slices % g == 0 && min_chunks * (n_slices / g) >= 2 * 256) return g;
  return 1;
}

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

hipError_t launch_ffn_up(int fmt, const uint16_t* x16, const int* sorted_slot, int k, int64_t S,
                         const Chunk* chunks, const int* n_chunks, int max_chunks_,
                         const void* gate_codes, const void* up_codes, const uint16_t* gate_scales,
                         const uint16_t* up_scales, int E, int H, int I, uint16_t* a16,
                         hipStream_t s) {
  (void)E;
  const int G = slices_per_unit(I / 128, 1, S);
  const int grid = grid_for_units((int64_t)max_chunks_ * (I / 128 / G));
  const uint8_t* gc = static_cast<const uint8_t*>(gate_codes);
  const uint8_t* uc = static_cast<const uint8_t*>(up_codes);
  allow_big_lds();
  if (fmt == 2)
    ffn_up_kernel<2><<<grid, kGemmThreads, kGemmLds, s>>>(x16, sorted_slot, k, chunks, n_chunks, gc,
                                                          uc, gate_scales, up_scales, H, I, G, a16);
  else
    ffn_up_kernel<3><<<grid, kGemmThreads, kGemmLds, s>>>(x16, sorted_slot, k, chunks, n_chunks, gc,
                                                          uc, gate_scales, up_scales, H, I, G, a16);
  return hipGetLastError();
}

hipError_t launch_ffn_down(int fmt, const uint16_t* a16, const int* sorted_slot, int64_t S,
                           const Chunk* chunks, const int* n_chunks, int max_chunks_,
                           const void* down_codes, const uint16_t* down_scales, int E, int H,
                           int I, uint16_t* expert_out, hipStream_t s) {
  (void)E;
  const int G = slices_per_unit(H / 256, 2, S);
  const int grid = grid_for_units((int64_t)max_chunks_ * (H / 256 / G));
  const uint8_t* dc = static_cast<const uint8_t*>(down_codes);
  allow_big_lds();
  if (fmt == 2)
    ffn_down_kernel<2><<<grid, kGemmThreads, kGemmLds, s>>>(a16, sorted_slot, chunks, n_chunks, dc,
                                                            down_scales, H, I, G, expert_out);
  else
    ffn_down_kernel<3><<<grid, kGemmThreads, kGemmLds, s>>>(a16, sorted_slot, chunks, n_chunks, dc,
                                                            down_scales, H, I, G, expert_out);
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
