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

}  // namespace

hipError_t mfma_probe(int workgroups, int iters, float *out, hipStream_t s) {
  OASES_LAUNCH(mfma_probe_kernel, dim3(workgroups), dim3(256), s, iters, out);
  return hipGetLastError();
}

}  // namespace oases
