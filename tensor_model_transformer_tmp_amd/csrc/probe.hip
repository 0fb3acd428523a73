// Dense bf16 matrix-core throughput probe: every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 on four independent accumulators (so no MFMA
// waits for the previous one's result), with operands held in registers and
// no memory traffic in the loop.  Its rate is the MFMA peak that the GEMM and
// attention kernels can be held against on this GPU.
#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8v a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
  }
  f32x16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the MFMAs live
}

// Operand feed probe: each workgroup (4 waves) cycles through its own 64 KB
// slice of an L2-resident source, one 1 KB unit per wave instruction, either
// by the LDS DMA the GEMM loaders use (mode 0), by global loads into VGPRs
// (mode 1), or by global loads followed by LDS writes (mode 2).  Its rate is
// what one CU can take in from the cache hierarchy per path.
constexpr int FEED_SLICE = 64 << 10;

template <int MODE>
__global__ void __launch_bounds__(256)
    feed_probe_kernel(const char *__restrict__ src, int64_t src_bytes, uint32_t *__restrict__ out, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[FEED_SLICE];
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // slice [off, off + 64 KB) lies in the source (its size is a multiple of 64 KB)
  const char *base = src + ((int64_t)blockIdx.x * FEED_SLICE) % src_bytes;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint32_t l0 = lds_addr(lds);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t unit = (uint32_t)((i * 8 + u) * 4 + wave) % (FEED_SLICE / 1024);
      const uint32_t off = unit * 1024 + lane * 16;
      if constexpr (MODE == 0) {
        dma16_s(base, off, l0 + unit * 1024);
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(base + off);
        if constexpr (MODE == 1) acc ^= v;
        else *reinterpret_cast<u32x4 *>(lds + off) = v;
      }
    }
    if constexpr (MODE == 0) wait_vmcnt<8>();
  }
  if constexpr (MODE == 0) wait_vmcnt<0>();
  __syncthreads();
  if constexpr (MODE != 1) acc ^= *reinterpret_cast<const u32x4 *>(lds + threadIdx.x * 16);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t feed_probe(int mode, int workgroups, int iters, const void *src, int64_t src_bytes, uint32_t *out,
                      hipStream_t s) {
  const char *p = static_cast<const char *>(src);
  switch (mode) {
    case 0: OASES_LAUNCH(feed_probe_kernel<0>, dim3(workgroups), dim3(256), s, p, src_bytes, out, iters); break;
    case 1: OASES_LAUNCH(feed_probe_kernel<1>, dim3(workgroups), dim3(256), s, p, src_bytes, out, iters); break;
    case 2: OASES_LAUNCH(feed_probe_kernel<2>, dim3(workgroups), dim3(256), s, p, src_bytes, out, iters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t mfma_probe(int workgroups, int iters, float *out, hipStream_t s) {
  OASES_LAUNCH(mfma_probe_kernel, dim3(workgroups), dim3(256), s, iters, out);
  return hipGetLastError();
}

}  // namespace oases
