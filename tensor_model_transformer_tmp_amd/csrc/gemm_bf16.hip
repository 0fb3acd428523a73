// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), float32
// accumulation, LDS double-buffered 64-deep k tiles.
//
// Used for the column-parallel and row-parallel GEMMs of a TMP shard and for
// their data and weight gradients:
//   forward / recompute   C[T, N] = X[T, K] W[N, K]^T        (A KC, B KC)
//   data gradient         dX[T, K] = dC[T, N] W[N, K]         (A KC, B MC)
//   weight gradient       dW[N, K] = dC[T, N]^T X[T, K]       (A MC, B MC)
//
// Tiling: a workgroup computes a BM x BN tile of C with WGM x WGN waves.
// Every operand tile is staged in LDS as [rows][64 + 8] bf16 with k
// contiguous, so each MFMA fragment is one 16-byte LDS read.  Operands whose
// contiguous dimension is not k (MC) are transposed in registers (8x8 bf16
// blocks) on their way into LDS.  The MFMA computes the transposed tile
// C^T = B^T A^T, so a lane owns one row m of C and runs of four consecutive
// columns n, which the epilogue writes as 8- or 16-byte vectors.
#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in bf16 (144 bytes: conflict-free 16-byte reads)

template <int ROWS, int NT, Layout LAY>
struct TileLoader {
  // KC: ROWS*8 16-byte chunks; MC: ROWS 8x8 blocks (8 loads each)
  static constexpr int ITEMS = (LAY == KC) ? (ROWS * 8 + NT - 1) / NT : (ROWS + NT - 1) / NT;
  static constexpr int REGS = (LAY == KC) ? ITEMS : ITEMS * 8;
  uint4 r[REGS];

  // rows_total: extent of the row dimension of the tile's matrix (M or N)
  __device__ __forceinline__ void load(const bf16_t *__restrict__ p, int ld, int row0,
                                       int rows_total, int k0, int K, int tid) {
    if constexpr (LAY == KC) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int c = tid + i * NT;
        const int row = c >> 3, kc = c & 7;
        const int gr = row0 + row, gk = k0 + kc * 8;
        const bool ok = (c < ROWS * 8) && gr < rows_total && gk < K;
        r[i] = ok ? *reinterpret_cast<const uint4 *>(p + (int64_t)gr * ld + gk)
                  : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int b = tid + i * NT;
        const int kb = b & 7, rb = b >> 3;
        const int gc = row0 + rb * 8;
        const bool okc = (b < ROWS) && gc < rows_total;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int gk = k0 + kb * 8 + q;
          r[i * 8 + q] = (okc && gk < K)
                             ? *reinterpret_cast<const uint4 *>(p + (int64_t)gk * ld + gc)
                             : make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16_t *__restrict__ s, int tid) {
    if constexpr (LAY == KC) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int c = tid + i * NT;
        if (c < ROWS * 8) {
          const int row = c >> 3, kc = c & 7;
          *reinterpret_cast<uint4 *>(s + row * LDK + kc * 8) = r[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int b = tid + i * NT;
        if (b < ROWS) {
          const int kb = b & 7, rb = b >> 3;
          uint4 blk[8], t[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) blk[q] = r[i * 8 + q];
          transpose8x8_bf16(blk, t);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint4 *>(s + (rb * 8 + j) * LDK + kb * 8) = t[j];
        }
      }
    }
  }
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int BM, int BN, int WGM, int WGN, Layout LA, Layout LB, int EPI>
__global__ void __launch_bounds__(WGM *WGN * 64)
    gemm_bf16_kernel(GemmArgs g) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must be a multiple of 32");
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;  // hl: which 32-lane half
  const int wm = wave % WGM, wn = wave / WGM;

  // tile order: consecutive workgroups of one XCD (ids i, i+8, ...) take
  // neighbouring tiles, grouped 8 m-tiles at a time along n for L2 reuse
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  constexpr int GROUP = 8;
  const int group_span = GROUP * tiles_n;
  const int grp = bid / group_span;
  const int first_m = grp * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % group_span) % gsize;
  const int tn = (bid % group_span) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t *__restrict__ A = static_cast<const bf16_t *>(g.A);
  const bf16_t *__restrict__ B = static_cast<const bf16_t *>(g.B);
  TileLoader<BM, NT, LA> la;
  TileLoader<BN, NT, LB> lb;

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  const int nk = (g.K + BK - 1) / BK;
  la.load(A, g.lda, m0, g.M, 0, g.K, tid);
  lb.load(B, g.ldb, n0, g.N, 0, g.K, tid);
  la.store(sA[0], tid);
  lb.store(sB[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, g.lda, m0, g.M, (kt + 1) * BK, g.K, tid);
      lb.load(B, g.ldb, n0, g.N, (kt + 1) * BK, g.K, tid);
    }
    const bf16_t *a_s = sA[buf] + (wm * WTM + l32) * LDK + hl * 8;
    const bf16_t *b_s = sB[buf] + (wn * WTN + l32) * LDK + hl * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 xa[TM], wb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        xa[i] = *reinterpret_cast<const bf16x8 *>(a_s + i * 32 * LDK + ks * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        wb[j] = *reinterpret_cast<const bf16x8 *>(b_s + j * 32 * LDK + ks * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[j][i] = mfma32(wb[j], xa[i], acc[j][i]);
    }
    if (more) {
      la.store(sA[buf ^ 1], tid);
      lb.store(sB[buf ^ 1], tid);
    }
    __syncthreads();
  }

  // epilogue: acc[j][i][jj*4 + ii] is C[m][n] with
  //   m = m0 + wm*WTM + i*32 + l32,  n = n0 + wn*WTN + j*32 + jj*8 + hl*4 + ii
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WTM + i * 32 + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = n0 + wn * WTN + j * 32 + jj * 8 + hl * 4;
        if (n >= g.N) continue;
        float v[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[ii] = acc[j][i][jj * 4 + ii];
        if constexpr (EPI == EPI_F32) {
          float *c = static_cast<float *>(g.C) + (int64_t)m * g.ldc + n;
          float4 o = make_float4(v[0], v[1], v[2], v[3]);
          if (g.beta) {
            const float4 old = *reinterpret_cast<const float4 *>(c);
            o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
          }
          *reinterpret_cast<float4 *>(c) = o;
        } else {
          if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
            const uint2 bb = *reinterpret_cast<const uint2 *>(
                static_cast<const bf16_t *>(g.bias) + n);
            v[0] += lo_f32(bb.x); v[1] += hi_f32(bb.x);
            v[2] += lo_f32(bb.y); v[3] += hi_f32(bb.y);
          }
          if constexpr (EPI == EPI_BIAS_GELU) {
            if (g.pre) {
              *reinterpret_cast<uint2 *>(static_cast<bf16_t *>(g.pre) + (int64_t)m * g.ld_pre + n) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) v[ii] = gelu_f(v[ii]);
          }
          if constexpr (EPI == EPI_GELU_BWD) {
            const uint2 uu = *reinterpret_cast<const uint2 *>(
                static_cast<const bf16_t *>(g.aux) + (int64_t)m * g.ld_aux + n);
            v[0] *= gelu_grad_f(lo_f32(uu.x)); v[1] *= gelu_grad_f(hi_f32(uu.x));
            v[2] *= gelu_grad_f(lo_f32(uu.y)); v[3] *= gelu_grad_f(hi_f32(uu.y));
          }
          *reinterpret_cast<uint2 *>(static_cast<bf16_t *>(g.C) + (int64_t)m * g.ldc + n) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, Layout LA, Layout LB, int EPI>
hipError_t launch(const GemmArgs &g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, LA, LB, EPI>), dim3(tiles),
                     dim3(WGM * WGN * 64), 0, s, g);
  return hipGetLastError();
}

template <Layout LA, Layout LB, int EPI>
hipError_t dispatch_tile(const GemmArgs &g, hipStream_t s) {
  // Large tiles when they alone fill the chip; otherwise 128x128 tiles.
  const int64_t big_tiles = (int64_t)((g.M + 255) / 256) * ((g.N + 127) / 128);
  if (big_tiles >= 256) return launch<256, 128, 2, 2, LA, LB, EPI>(g, s);
  return launch<128, 128, 2, 2, LA, LB, EPI>(g, s);
}

}  // namespace

hipError_t gemm_bf16(Layout la, Layout lb, Epi epi, const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (la == KC && lb == KC) {
    switch (epi) {
      case EPI_STORE: return dispatch_tile<KC, KC, EPI_STORE>(g, s);
      case EPI_BIAS: return dispatch_tile<KC, KC, EPI_BIAS>(g, s);
      case EPI_BIAS_GELU: return dispatch_tile<KC, KC, EPI_BIAS_GELU>(g, s);
      default: break;
    }
  } else if (la == KC && lb == MC) {
    switch (epi) {
      case EPI_STORE: return dispatch_tile<KC, MC, EPI_STORE>(g, s);
      case EPI_GELU_BWD: return dispatch_tile<KC, MC, EPI_GELU_BWD>(g, s);
      default: break;
    }
  } else if (la == MC && lb == MC) {
    if (epi == EPI_F32) return dispatch_tile<MC, MC, EPI_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace oases
