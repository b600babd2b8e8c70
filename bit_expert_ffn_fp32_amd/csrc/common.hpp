// Device helpers shared by the gfx950 kernels of the MoE expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define STRATA_DEVICE __device__ __forceinline__

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace strata {

constexpr int kWave = 64;

STRATA_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
STRATA_DEVICE uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp16 bit pattern -> fp32 (exact; the hardware conversion handles subnormals).
STRATA_DEVICE float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// (value, index) arg-max with ties to the lower index, across the 64 lanes of a wave.
STRATA_DEVICE void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off);
    int oi = __shfl_xor(i, off);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

STRATA_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

STRATA_DEVICE int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace strata
