// Causal multi-head attention of the attention block's shard (bf16, MFMA).
//
// QKV is [nb*s, 3a] with columns [Q | K | V], each head-major (head h owns
// columns h*d .. h*d+d-1 of its part).  O is [nb*s, a].  Per (sequence, head):
//   O = softmax(Q K^T / sqrt(d) + causal mask) V,  lse = log sum exp of a row.
//
// Forward: a workgroup owns 128 queries (4 waves x 32).  Each wave keeps its
// Q fragments in registers and walks 64-key blocks staged in LDS (K as
// [key][d], V transposed as [d][key]).  It computes S^T = K Q^T so that a
// lane owns one query and 16 keys of the 32x32 MFMA tile: the row max and
// row sum of the online softmax are then a per-lane reduction plus one
// exchange with the lane 32 away (a wavefront reduction), and the softmax
// rescale of O^T is a per-lane scalar.  The P^T tile in accumulator layout is
// directly the B operand of O^T += V^T P^T once V^T is read with the same key
// permutation.
//
// Backward (no atomics): delta = rowsum(dO * O); a dK/dV kernel owns 128 keys
// and walks query blocks (S = Q K^T, dP = dO V^T, dV^T += dO^T P,
// dK^T += Q^T dS); a dQ kernel owns 128 queries and walks key blocks
// (S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T).  P is rebuilt from lse.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

constexpr int NT = 256;       // 4 waves
constexpr int WQ = 32;        // rows per wave
constexpr int TILE = 128;     // rows per workgroup
constexpr int BLK = 64;       // rows per staged block
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_frag(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 load_frag(const bf16_t *p) {
  return as_frag(*reinterpret_cast<const uint4 *>(p));
}

// accumulator registers [8h, 8h+8) -> bf16 B-operand fragment
__device__ __forceinline__ bf16x8 acc_to_frag(const f32x16 &a, int h) {
  return as_frag(make_uint4(pack_bf16x2(a[8 * h + 0], a[8 * h + 1]), pack_bf16x2(a[8 * h + 2], a[8 * h + 3]),
                            pack_bf16x2(a[8 * h + 4], a[8 * h + 5]), pack_bf16x2(a[8 * h + 6], a[8 * h + 7])));
}

// A-operand fragment from a transposed LDS tile sT[d][rows] whose k index runs
// over rows in the accumulator-row order: elements 0..3 are rows c0+g*4+0..3,
// elements 4..7 rows c0+8+g*4+0..3 (c0 = 32*sub + 16*half).
__device__ __forceinline__ bf16x8 load_perm_frag(const bf16_t *sT, int pitch, int d, int c0, int g) {
  const uint2 lo = *reinterpret_cast<const uint2 *>(sT + d * pitch + c0 + g * 4);
  const uint2 hi = *reinterpret_cast<const uint2 *>(sT + d * pitch + c0 + 8 + g * 4);
  return as_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Stage rows [row0, row0+BLK) x D of a matrix with row stride ld into LDS as
// [BLK][D+8] (native) and/or [D][BLK+8] (transposed); rows >= nvalid are zero.
template <int D, bool NATIVE, bool TRANS>
__device__ __forceinline__ void stage(bf16_t *sn, bf16_t *st, const bf16_t *__restrict__ g, int ld,
                                      int row0, int nvalid, int tid) {
  if constexpr (NATIVE) {
    for (int c = tid; c < BLK * D / 8; c += NT) {
      const int r = c / (D / 8), dc = c % (D / 8);
      const int gr = row0 + r;
      const uint4 v = gr < nvalid ? *reinterpret_cast<const uint4 *>(g + (int64_t)gr * ld + dc * 8)
                                  : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(sn + r * (D + 8) + dc * 8) = v;
    }
  }
  if constexpr (TRANS) {
    for (int b = tid; b < (BLK / 8) * (D / 8); b += NT) {
      const int rb = b % (BLK / 8), dbk = b / (BLK / 8);
      uint4 rr[8], tt[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int gr = row0 + rb * 8 + q;
        rr[q] = gr < nvalid ? *reinterpret_cast<const uint4 *>(g + (int64_t)gr * ld + dbk * 8)
                            : make_uint4(0, 0, 0, 0);
      }
      transpose8x8_bf16(rr, tt);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint4 *>(st + (dbk * 8 + j) * (BLK + 8) + rb * 8) = tt[j];
    }
  }
}

// row index (within a 32-row MFMA tile) held in accumulator register r by lane group g
__device__ __forceinline__ int acc_row(int r, int g) { return (r >> 2) * 8 + g * 4 + (r & 3); }

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(NT)
    attn_fwd_kernel(const bf16_t *__restrict__ qkv, bf16_t *__restrict__ out, float *__restrict__ lse,
                    int s, int nh, int causal, float scale_log2) {
  constexpr int PK = D + 8, PV = BLK + 8;
  __shared__ __attribute__((aligned(16))) bf16_t sK[BLK * PK];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[D * PV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int ntile = (s + TILE - 1) / TILE;
  const int q0 = (ntile - 1 - (int)blockIdx.x) * TILE;  // heaviest causal tiles first
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const int qw = q0 + wave * WQ, qi = qw + l32;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = qi < s ? load_frag(Qp + (int64_t)qi * ld + kk * 16 + g * 8) : as_frag(make_uint4(0, 0, 0, 0));
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = causal ? min(s, q0 + TILE) : s;
  for (int kb0 = 0; kb0 < kend; kb0 += BLK) {
    __syncthreads();
    stage<D, true, false>(sK, nullptr, Kp, ld, kb0, s, tid);
    stage<D, false, true>(nullptr, sVt, Vp, ld, kb0, s, tid);
    __syncthreads();
    if (qw >= s || (causal && kb0 > qw + WQ - 1)) continue;

    f32x16 st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[sub][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        st[sub] = mfma32(load_frag(sK + (sub * 32 + l32) * PK + kk * 16 + g * 8), qf[kk], st[sub]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + sub * 32 + acc_row(r, g);
        float x = st[sub][r] * scale_log2;
        if (key >= s || (causal && key > qi)) x = -INFINITY;
        st[sub][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - base);
    float rs = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(st[sub][r] - base);
        st[sub][r] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
    bf16x8 pf[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pf[sub * 2 + hh] = acc_to_frag(st[sub], hh);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        oacc[t] = mfma32(load_perm_frag(sVt, PV, t * 32 + l32, c * 16, g), pf[c], oacc[t]);
  }

  if (qi < s) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16_t *op = out + (int64_t)(b * s + qi) * a + h * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = t * 32 + jj * 8 + g * 4;
        *reinterpret_cast<uint2 *>(op + d0) =
            make_uint2(pack_bf16x2(oacc[t][jj * 4 + 0] * inv, oacc[t][jj * 4 + 1] * inv),
                       pack_bf16x2(oacc[t][jj * 4 + 2] * inv, oacc[t][jj * 4 + 3] * inv));
      }
    if (g == 0) lse[(int64_t)bh * s + qi] = (m_run + log2f(l_run)) * 0.69314718055994531f;
  }
}

// ---------------------------------------------------------------------------
// backward: delta = rowsum(dO * O) per (sequence, head, query)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
    attn_delta_kernel(const bf16_t *__restrict__ o, const bf16_t *__restrict__ dout,
                      float *__restrict__ delta, int nb, int s, int nh) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, t, h), h fastest
  if (idx >= (int64_t)nb * s * nh) return;
  const int h = idx % nh;
  const int64_t row = idx / nh;  // b*s + t
  const int a = nh * D;
  const bf16_t *po = o + row * a + h * D, *pd = dout + row * a + h * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    const uint4 x = *reinterpret_cast<const uint4 *>(po + c);
    const uint4 y = *reinterpret_cast<const uint4 *>(pd + c);
    acc += lo_f32(x.x) * lo_f32(y.x) + hi_f32(x.x) * hi_f32(y.x) + lo_f32(x.y) * lo_f32(y.y) +
           hi_f32(x.y) * hi_f32(y.y) + lo_f32(x.z) * lo_f32(y.z) + hi_f32(x.z) * hi_f32(y.z) +
           lo_f32(x.w) * lo_f32(y.w) + hi_f32(x.w) * hi_f32(y.w);
  }
  const int b = (int)(row / s), t = (int)(row % s);
  delta[((int64_t)b * nh + h) * s + t] = acc;
}

// ---------------------------------------------------------------------------
// backward: dK, dV.  A wave owns 32 keys; queries are walked in 64-row blocks.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(NT)
    attn_bwd_dkdv_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                         const float *__restrict__ lse, const float *__restrict__ delta,
                         bf16_t *__restrict__ dqkv, int s, int nh, int causal, float scale_log2,
                         float scale) {
  constexpr int PN = D + 8, PT = BLK + 8;
  __shared__ __attribute__((aligned(16))) bf16_t sQ[BLK * PN];
  __shared__ __attribute__((aligned(16))) bf16_t sdO[BLK * PN];
  __shared__ __attribute__((aligned(16))) bf16_t sQt[D * PT];
  __shared__ __attribute__((aligned(16))) bf16_t sdOt[D * PT];
  __shared__ float sL[BLK], sDl[BLK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int k0 = blockIdx.x * TILE;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const float *lp = lse + (int64_t)bh * s, *dp = delta + (int64_t)bh * s;
  const int kw = k0 + wave * WQ, kj = kw + l32;

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bool ok = kj < s;
    kf[kk] = ok ? load_frag(Kp + (int64_t)kj * ld + kk * 16 + g * 8) : as_frag(make_uint4(0, 0, 0, 0));
    vf[kk] = ok ? load_frag(Vp + (int64_t)kj * ld + kk * 16 + g * 8) : as_frag(make_uint4(0, 0, 0, 0));
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dv[t][r] = 0.f; dk[t][r] = 0.f; }

  const int qstart = causal ? (k0 / BLK) * BLK : 0;
  for (int qb0 = qstart; qb0 < s; qb0 += BLK) {
    __syncthreads();
    stage<D, true, true>(sQ, sQt, Qp, ld, qb0, s, tid);
    stage<D, true, true>(sdO, sdOt, dOp, a, qb0, s, tid);
    if (tid < BLK) {
      const int q = qb0 + tid;
      sL[tid] = q < s ? lp[q] * LOG2E : INFINITY;  // P = 0 for rows past the end
      sDl[tid] = q < s ? dp[q] : 0.f;
    }
    __syncthreads();
    if (kw >= s || (causal && kw > qb0 + BLK - 1)) continue;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (causal && kw > qb0 + sub * 32 + 31) continue;
      f32x16 sacc, dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; dpacc[r] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc = mfma32(load_frag(sQ + (sub * 32 + l32) * PN + kk * 16 + g * 8), kf[kk], sacc);
        dpacc = mfma32(load_frag(sdO + (sub * 32 + l32) * PN + kk * 16 + g * 8), vf[kk], dpacc);
      }
      // sacc[r]: S[q][key] with q = qb0 + sub*32 + acc_row(r, g), key = kj
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = sub * 32 + acc_row(r, g);
        const int q = qb0 + ql;
        float p = exp2f(sacc[r] * scale_log2 - sL[ql]);
        if (causal && kj > q) p = 0.f;
        sacc[r] = p;
        dpacc[r] = p * (dpacc[r] - sDl[ql]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8 pfr = acc_to_frag(sacc, hh), dsf = acc_to_frag(dpacc, hh);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          dv[t] = mfma32(load_perm_frag(sdOt, PT, t * 32 + l32, sub * 32 + hh * 16, g), pfr, dv[t]);
          dk[t] = mfma32(load_perm_frag(sQt, PT, t * 32 + l32, sub * 32 + hh * 16, g), dsf, dk[t]);
        }
      }
    }
  }
  if (kj < s) {
    bf16_t *pk = dqkv + (int64_t)(b * s + kj) * ld + a + h * D;
    bf16_t *pv = pk + a;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = t * 32 + jj * 8 + g * 4;
        *reinterpret_cast<uint2 *>(pk + d0) =
            make_uint2(pack_bf16x2(dk[t][jj * 4 + 0] * scale, dk[t][jj * 4 + 1] * scale),
                       pack_bf16x2(dk[t][jj * 4 + 2] * scale, dk[t][jj * 4 + 3] * scale));
        *reinterpret_cast<uint2 *>(pv + d0) =
            make_uint2(pack_bf16x2(dv[t][jj * 4 + 0], dv[t][jj * 4 + 1]),
                       pack_bf16x2(dv[t][jj * 4 + 2], dv[t][jj * 4 + 3]));
      }
  }
}

// ---------------------------------------------------------------------------
// backward: dQ.  A wave owns 32 queries; keys are walked in 64-row blocks.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(NT)
    attn_bwd_dq_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                       const float *__restrict__ lse, const float *__restrict__ delta,
                       bf16_t *__restrict__ dqkv, int s, int nh, int causal, float scale_log2,
                       float scale) {
  constexpr int PN = D + 8, PT = BLK + 8;
  __shared__ __attribute__((aligned(16))) bf16_t sK[BLK * PN];
  __shared__ __attribute__((aligned(16))) bf16_t sV[BLK * PN];
  __shared__ __attribute__((aligned(16))) bf16_t sKt[D * PT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int ntile = (s + TILE - 1) / TILE;
  const int q0 = (ntile - 1 - (int)blockIdx.x) * TILE;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const int qw = q0 + wave * WQ, qi = qw + l32;
  const bool qok = qi < s;

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qok ? load_frag(Qp + (int64_t)qi * ld + kk * 16 + g * 8) : as_frag(make_uint4(0, 0, 0, 0));
    df[kk] = qok ? load_frag(dOp + (int64_t)qi * a + kk * 16 + g * 8) : as_frag(make_uint4(0, 0, 0, 0));
  }
  const float lq = qok ? lse[(int64_t)bh * s + qi] * LOG2E : INFINITY;
  const float dq_delta = qok ? delta[(int64_t)bh * s + qi] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[t][r] = 0.f;

  const int kend = causal ? min(s, q0 + TILE) : s;
  for (int kb0 = 0; kb0 < kend; kb0 += BLK) {
    __syncthreads();
    stage<D, true, true>(sK, sKt, Kp, ld, kb0, s, tid);
    stage<D, true, false>(sV, nullptr, Vp, ld, kb0, s, tid);
    __syncthreads();
    if (qw >= s || (causal && kb0 > qw + WQ - 1)) continue;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; dpacc[r] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc = mfma32(load_frag(sK + (sub * 32 + l32) * PN + kk * 16 + g * 8), qf[kk], sacc);
        dpacc = mfma32(load_frag(sV + (sub * 32 + l32) * PN + kk * 16 + g * 8), df[kk], dpacc);
      }
      // sacc[r]: S^T[key][q] with key = kb0 + sub*32 + acc_row(r, g), q = qi
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + sub * 32 + acc_row(r, g);
        float p = exp2f(sacc[r] * scale_log2 - lq);
        if (key >= s || (causal && key > qi)) p = 0.f;
        dpacc[r] = p * (dpacc[r] - dq_delta);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8 dsf = acc_to_frag(dpacc, hh);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          dq[t] = mfma32(load_perm_frag(sKt, PT, t * 32 + l32, sub * 32 + hh * 16, g), dsf, dq[t]);
      }
    }
  }
  if (qok) {
    bf16_t *pq = dqkv + (int64_t)(b * s + qi) * ld + h * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = t * 32 + jj * 8 + g * 4;
        *reinterpret_cast<uint2 *>(pq + d0) =
            make_uint2(pack_bf16x2(dq[t][jj * 4 + 0] * scale, dq[t][jj * 4 + 1] * scale),
                       pack_bf16x2(dq[t][jj * 4 + 2] * scale, dq[t][jj * 4 + 3] * scale));
      }
  }
}

template <int D>
hipError_t fwd_d(int nb, int s, int nh, int causal, const void *qkv, void *o, float *lse, hipStream_t st) {
  dim3 grid((s + TILE - 1) / TILE, nb * nh);
  const float scale_log2 = LOG2E / sqrtf((float)D);
  hipLaunchKernelGGL(attn_fwd_kernel<D>, grid, dim3(NT), 0, st, static_cast<const bf16_t *>(qkv),
                     static_cast<bf16_t *>(o), lse, s, nh, causal, scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(int nb, int s, int nh, int causal, const void *qkv, const void *o, const void *dout,
                 const float *lse, float *delta, void *dqkv, hipStream_t st) {
  const int64_t rows = (int64_t)nb * s * nh;
  hipLaunchKernelGGL(attn_delta_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st,
                     static_cast<const bf16_t *>(o), static_cast<const bf16_t *>(dout), delta, nb, s, nh);
  const float scale = 1.f / sqrtf((float)D), scale_log2 = scale * LOG2E;
  dim3 grid((s + TILE - 1) / TILE, nb * nh);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, grid, dim3(NT), 0, st, static_cast<const bf16_t *>(qkv),
                     static_cast<const bf16_t *>(dout), lse, delta, static_cast<bf16_t *>(dqkv), s, nh,
                     causal, scale_log2, scale);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, grid, dim3(NT), 0, st, static_cast<const bf16_t *>(qkv),
                     static_cast<const bf16_t *>(dout), lse, delta, static_cast<bf16_t *>(dqkv), s, nh,
                     causal, scale_log2, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t attention_fwd(int nb, int s, int nh, int d, int causal, const void *qkv, void *o,
                         float *lse, hipStream_t st) {
  if (nb <= 0 || s <= 0 || nh <= 0) return hipSuccess;
  if (d == 64) return fwd_d<64>(nb, s, nh, causal, qkv, o, lse, st);
  if (d == 128) return fwd_d<128>(nb, s, nh, causal, qkv, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t attention_bwd(int nb, int s, int nh, int d, int causal, const void *qkv, const void *o,
                         const void *dout, const float *lse, float *delta, void *dqkv, hipStream_t st) {
  if (nb <= 0 || s <= 0 || nh <= 0) return hipSuccess;
  if (d == 64) return bwd_d<64>(nb, s, nh, causal, qkv, o, dout, lse, delta, dqkv, st);
  if (d == 128) return bwd_d<128>(nb, s, nh, causal, qkv, o, dout, lse, delta, dqkv, st);
  return hipErrorInvalidValue;
}

}  // namespace oases
