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

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 64x64 -> 128-bit products on the 4-word counter, key bumped by the Weyl
// constants after each round.  The counter is replaced by the output.
__device__ __forceinline__ void philox4x64(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// Dropout + residual of the 8 elements of vector v (elements 8v .. 8v+7 of a
// sub-batch buffer): acc[e] = res[e] + (kept ? acc[e] * scale : 0), one fused
// multiply-add, so every kernel that applies it gets the same bits.
__device__ __forceinline__ void drop_res8(float (&acc)[8], uint4 res, int64_t v, uint64_t seed,
                                          uint64_t layer, uint64_t sb, uint64_t thr, float scale,
                                          bool drop) {
  const float r[8] = {lo_f32(res.x), hi_f32(res.x), lo_f32(res.y), hi_f32(res.y),
                      lo_f32(res.z), hi_f32(res.z), lo_f32(res.w), hi_f32(res.w)};
  if (!drop) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(acc[e], 1.f, r[e]);
    return;
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint64_t c[4] = {(uint64_t)(2 * v + hh), sb, 0ull, 0ull};
    philox4x64(c, seed, layer);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * hh + j;
      acc[e] = c[j] < thr ? __builtin_fmaf(acc[e], scale, r[e]) : r[e];
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// 64 zero bytes in global memory: the source of DMA lanes whose element lies
// outside a matrix, so partial tiles are filled with exact zeros.
__device__ __forceinline__ const bf16_t *zero_page() {
  static __device__ __attribute__((aligned(64))) bf16_t page[32];  // zero-initialised
  return page;
}

// One LDS-DMA instruction (gfx950 global_load_lds_dwordx4): every lane copies
// 16 bytes from its global address; the wave's 64 x 16 bytes land
// contiguously at the LDS address `dst` (through M0).  Issued as inline asm
// so that the compiler's memory model does not treat the DMA as a pending LDS
// store (a fenced barrier would otherwise drain all outstanding DMA before
// every tile); completion is awaited explicitly with wait_vmcnt().
__device__ __forceinline__ void dma16(const bf16_t *src, const bf16_t *dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_t *)dst;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
               : "m0", "memory");
}

// LDS byte address of a shared-memory pointer (one address-space cast; the
// DMA helpers below take 32-bit LDS addresses so that per-unit address
// arithmetic stays in 32-bit scalar registers).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)p);
}

// DMA of one 1-KB unit with a scalar base and a per-lane 32-bit byte offset
// (global_load_lds_dwordx4 v_off, s[base]): the 64 lanes' 16 bytes land
// contiguously at LDS byte address lds.
__device__ __forceinline__ void dma16_s(const void *base, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;  // uniform; made scalar explicitly
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sb)
               : "m0", "memory");
}
// the same with a per-lane 64-bit source address
__device__ __forceinline__ void dma16_v(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
               : "m0", "memory");
}

// 16 bytes of LDS at a 32-bit LDS byte address
__device__ __forceinline__ bf16x8 lds_frag(uint32_t addr) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)addr);
}

// Chunk swizzle of a row-major bf16 tile read with ds_read_b64_tr_b16: a read
// covers 4 consecutive rows x 64 bytes per 32 lanes.  16-byte chunk c of row
// k is stored at c ^ mc_swz(k) so those rows land in distinct 64-byte
// quarters of the 256-byte bank space: rows of >= 256 bytes use (k & 3),
// 128-byte rows (two per bank window) use bit 1 of k.
template <int ROW_ELEMS>
__device__ __forceinline__ int mc_swz(int k) {
  static_assert(ROW_ELEMS == 64 || ROW_ELEMS % 128 == 0, "row length");
  return ROW_ELEMS == 64 ? (((k >> 1) & 1) << 2) : ((k & 3) << 2);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS only (global traffic needs no ordering
// across it: DMA completion is awaited with wait_vmcnt before it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// GeLU and its derivative in float32, gelu(u) = u * Phi(u) with the standard
// normal CDF Phi(u) = (1 + erf(u / sqrt 2)) / 2.  erf is evaluated with the
// rational-exponential approximation 7.1.26 of Abramowitz & Stegun (Handbook
// of Mathematical Functions): for x >= 0,
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x),  |error| <= 1.5e-7,
// which is below float32 resolution of Phi near 1 and far below bf16
// resolution.  The tail Q = 1 - erf(x) is formed directly (no cancellation)
// and its exp(-x^2) = exp(-u^2 / 2) is shared with the density in gelu'.
struct PhiParts {
  float phi_cdf;  // Phi(u)
  float pdf;      // phi(u) = exp(-u^2/2) / sqrt(2 pi)
};

__device__ __forceinline__ PhiParts normal_cdf_pdf(float u) {
  const float x = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-x * x * 1.4426950408889634f);  // exp(-x^2)
  const float half_q = 0.5f * poly * e;                                  // (1 - erf(x)) / 2
  PhiParts r;
  r.phi_cdf = u >= 0.f ? 1.0f - half_q : half_q;
  r.pdf = 0.39894228040143268f * e;
  return r;
}

__device__ __forceinline__ float gelu_f(float u) { return u * normal_cdf_pdf(u).phi_cdf; }

__device__ __forceinline__ float gelu_grad_f(float u) {
  const PhiParts p = normal_cdf_pdf(u);
  return fmaf(u, p.pdf, p.phi_cdf);
}

// GeLU, tanh form: gelu_t(u) = u/2 (1 + tanh(k)), k = sqrt(2/pi) (u + 0.044715 u^3);
// d/du = (1 + tanh k)/2 + u/2 (1 - tanh^2 k) sqrt(2/pi) (1 + 3 * 0.044715 u^2).
// tanh k = 1 - 2 / (1 + e^(2k)) with e^(2k) = 2^(2k log2 e) (v_exp_f32); the
// form saturates to +-1 for large |k| (e^(2k) -> inf or 0).
__device__ __forceinline__ float tanh_of(float k) {
  return 1.f - 2.f / (1.f + __builtin_amdgcn_exp2f(k * 2.8853900817779268f));  // 2 log2(e)
}
__device__ __forceinline__ float gelu_tanh_f(float u) {
  const float k = 0.7978845608028654f * fmaf(0.044715f * u, u * u, u);
  return 0.5f * u * (1.f + tanh_of(k));
}
__device__ __forceinline__ float gelu_tanh_grad_f(float u) {
  const float k = 0.7978845608028654f * fmaf(0.044715f * u, u * u, u);
  const float t = tanh_of(k);
  return 0.5f * (1.f + t) + 0.5f * u * (1.f - t * t) * 0.7978845608028654f * fmaf(0.134145f * u, u, 1.f);
}

}  // namespace oases
