// Shared device helpers for the gfx950 kernels of liboases_shard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oases {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// low / high bf16 of a packed word -> float
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Transpose an 8x8 block of bf16 held as 8 rows of uint4 (row i = r[i], 8
// elements each) into 8 columns: o[j] holds element j of r[0..7].
__device__ __forceinline__ void transpose8x8_bf16(const uint4 (&r)[8], uint4 (&o)[8]) {
  const uint32_t *rw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rw[i] = reinterpret_cast<const uint32_t *>(&r[i]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = rw[2 * p][j >> 1], b = rw[2 * p + 1][j >> 1];
      // even j: low halves of a and b; odd j: high halves
      w[p] = (j & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                     : __builtin_amdgcn_perm(b, a, 0x05040100u);
    }
    o[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// exact GeLU and its derivative in float32: gelu(u) = u * Phi(u)
__device__ __forceinline__ float gelu_f(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_f(float u) {
  return 0.5f * (1.0f + erff(u * 0.70710678118654752f)) +
         u * 0.39894228040143268f * expf(-0.5f * u * u);
}

}  // namespace oases
