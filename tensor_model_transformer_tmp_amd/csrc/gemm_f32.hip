// float32 GEMM for the float32 storage configuration (small shards; the
// path there is latency bound, so a plain LDS-tiled SIMT kernel is used).
// Same operand layouts and epilogues as the bf16 MFMA kernel.
#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

constexpr int TB = 64, TK = 16;

template <Layout LA, Layout LB, int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g) {
  __shared__ float sA[TK][TB + 4];
  __shared__ float sB[TK][TB + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const float *__restrict__ A = static_cast<const float *>(g.A);
  const float *__restrict__ B = static_cast<const float *>(g.B);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + i * 256;
      int m, k;
      if (LA == KC) { m = idx / TK; k = idx % TK; } else { k = idx / TB; m = idx % TB; }
      const int gm = m0 + m, gk = k0 + k;
      float v = 0.f;
      if (gm < g.M && gk < g.K) v = (LA == KC) ? A[(int64_t)gm * g.lda + gk] : A[(int64_t)gk * g.lda + gm];
      sA[k][m] = v;
      int n;
      if (LB == KC) { n = idx / TK; k = idx % TK; } else { k = idx / TB; n = idx % TB; }
      const int gn = n0 + n;
      const int gk2 = k0 + k;
      float w = 0.f;
      if (gn < g.N && gk2 < g.K) w = (LB == KC) ? B[(int64_t)gn * g.ldb + gk2] : B[(int64_t)gk2 * g.ldb + gn];
      sB[k][n] = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[k][ty * 4 + i]; b[i] = sB[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      float v = acc[i][j];
      float *c = static_cast<float *>(g.C) + (int64_t)m * g.ldc + n;
      if constexpr (EPI == EPI_F32) {
        *c = g.beta ? *c + v : v;
        continue;
      }
      if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) v += static_cast<const float *>(g.bias)[n];
      if constexpr (EPI == EPI_BIAS_GELU) {
        if (g.pre) static_cast<float *>(g.pre)[(int64_t)m * g.ld_pre + n] = v;
        v = gelu_f(v);
      }
      if constexpr (EPI == EPI_GELU_BWD)
        v *= gelu_grad_f(static_cast<const float *>(g.aux)[(int64_t)m * g.ld_aux + n]);
      *c = v;
    }
  }
}

template <Layout LA, Layout LB, int EPI>
hipError_t launch(const GemmArgs &g, hipStream_t s) {
  dim3 grid((g.N + TB - 1) / TB, (g.M + TB - 1) / TB);
  OASES_LAUNCH((gemm_f32_kernel<LA, LB, EPI>), grid, dim3(256), s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_f32(Layout la, Layout lb, Epi epi, const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (la == KC && lb == KC) {
    switch (epi) {
      case EPI_STORE: return launch<KC, KC, EPI_STORE>(g, s);
      case EPI_BIAS: return launch<KC, KC, EPI_BIAS>(g, s);
      case EPI_BIAS_GELU: return launch<KC, KC, EPI_BIAS_GELU>(g, s);
      default: break;
    }
  } else if (la == KC && lb == MC) {
    switch (epi) {
      case EPI_STORE: return launch<KC, MC, EPI_STORE>(g, s);
      case EPI_GELU_BWD: return launch<KC, MC, EPI_GELU_BWD>(g, s);
      default: break;
    }
  } else if (la == MC && lb == MC) {
    if (epi == EPI_F32) return launch<MC, MC, EPI_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace oases
