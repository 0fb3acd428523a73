// Bandwidth-bound kernels: the AllReduce-point sum and the deterministic
// column sum used for bias gradients.
#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

// ---------------------------------------------------------------------------
// AllReduce point (Oases, Section IV: the AllReduce output is the sum of its
// w inputs).  out = own + peer_1 + ... + peer_{w-1}, float32 adds in that
// order, one rounding to the storage type.  Each thread streams 8 elements
// (16 bytes of bf16) per input per iteration, so every input read is one
// coalesced 16-byte load and the w loads of an iteration are in flight
// together.
// ---------------------------------------------------------------------------
constexpr int SUM_NT = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// streaming 16-byte load that bypasses cache retention (each byte is read once)
__device__ __forceinline__ uint4 stream_load(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// NP peers (compile time) and UNROLL vectors per thread per iteration: all
// UNROLL * (NP + 1) loads of an iteration are issued before the first add,
// so a grid of a few workgroups per CU keeps enough bytes in flight for HBM.
template <int NP>
__global__ void __launch_bounds__(SUM_NT)
    allreduce_bf16_kernel(const uint4 *__restrict__ own, const bf16_t *__restrict__ peers,
                          int64_t peer_stride, uint4 *__restrict__ out, int64_t nvec, DropRes t) {
  constexpr int UNROLL = NP >= 4 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * SUM_NT;
  for (int64_t v0 = (int64_t)blockIdx.x * SUM_NT + threadIdx.x; v0 < nvec; v0 += stride * UNROLL) {
    uint4 x[NP + 1][UNROLL];
#pragma unroll
    for (int k = 0; k <= NP; ++k) {
      const uint4 *src = k == 0 ? own : reinterpret_cast<const uint4 *>(peers + (int64_t)(k - 1) * peer_stride);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t v = v0 + u * stride;
        x[k][u] = v < nvec ? stream_load(src + v) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t v = v0 + u * stride;
      if (v >= nvec) continue;
      float acc[8] = {lo_f32(x[0][u].x), hi_f32(x[0][u].x), lo_f32(x[0][u].y), hi_f32(x[0][u].y),
                      lo_f32(x[0][u].z), hi_f32(x[0][u].z), lo_f32(x[0][u].w), hi_f32(x[0][u].w)};
#pragma unroll
      for (int k = 1; k <= NP; ++k) {
        const uint4 b = x[k][u];
        acc[0] += lo_f32(b.x); acc[1] += hi_f32(b.x); acc[2] += lo_f32(b.y); acc[3] += hi_f32(b.y);
        acc[4] += lo_f32(b.z); acc[5] += hi_f32(b.z); acc[6] += lo_f32(b.w); acc[7] += hi_f32(b.w);
      }
      if (t.res)
        drop_res8(acc, reinterpret_cast<const uint4 *>(t.res)[v], v, t.seed, t.layer, t.sb, t.thr, t.scale,
                  t.drop);
      out[v] = make_uint4(cvt_pk(acc[0], acc[1]), cvt_pk(acc[2], acc[3]), cvt_pk(acc[4], acc[5]),
                          cvt_pk(acc[6], acc[7]));
    }
  }
}

// Lean form of the same sum: one vector per thread per iteration, its NP + 1
// loads in flight, so few registers that its waves fit on a CU beside a
// GEMM workgroup's (the GEMM holds most of the register file but leaves the
// memory pipeline mostly idle).  Same adds in the same order: bit-identical.
template <int NP, bool TAIL>
__global__ void __launch_bounds__(SUM_NT)
    allreduce_bf16_lean_kernel(const uint4 *__restrict__ own, const bf16_t *__restrict__ peers,
                               int64_t peer_stride, uint4 *__restrict__ out, int64_t nvec, DropRes t) {
  for (int64_t v = (int64_t)blockIdx.x * SUM_NT + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * SUM_NT) {
    uint4 x[NP + 1];
#pragma unroll
    for (int k = 0; k <= NP; ++k) {
      const uint4 *src = k == 0 ? own : reinterpret_cast<const uint4 *>(peers + (int64_t)(k - 1) * peer_stride);
      x[k] = stream_load(src + v);
    }
    float acc[8] = {lo_f32(x[0].x), hi_f32(x[0].x), lo_f32(x[0].y), hi_f32(x[0].y),
                    lo_f32(x[0].z), hi_f32(x[0].z), lo_f32(x[0].w), hi_f32(x[0].w)};
#pragma unroll
    for (int k = 1; k <= NP; ++k) {
      const uint4 b = x[k];
      acc[0] += lo_f32(b.x); acc[1] += hi_f32(b.x); acc[2] += lo_f32(b.y); acc[3] += hi_f32(b.y);
      acc[4] += lo_f32(b.z); acc[5] += hi_f32(b.z); acc[6] += lo_f32(b.w); acc[7] += hi_f32(b.w);
    }
    if constexpr (TAIL)
      drop_res8(acc, reinterpret_cast<const uint4 *>(t.res)[v], v, t.seed, t.layer, t.sb, t.thr, t.scale, t.drop);
    out[v] = make_uint4(cvt_pk(acc[0], acc[1]), cvt_pk(acc[2], acc[3]), cvt_pk(acc[4], acc[5]),
                        cvt_pk(acc[6], acc[7]));
  }
}

// more peers than the unrolled kernels cover: a runtime loop over the peers
__global__ void __launch_bounds__(SUM_NT)
    allreduce_bf16_many_kernel(const uint4 *__restrict__ own, const bf16_t *__restrict__ peers,
                               int64_t peer_stride, int n_peers, uint4 *__restrict__ out, int64_t nvec,
                               DropRes t) {
  for (int64_t v = (int64_t)blockIdx.x * SUM_NT + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * SUM_NT) {
    const uint4 a = stream_load(own + v);
    float acc[8] = {lo_f32(a.x), hi_f32(a.x), lo_f32(a.y), hi_f32(a.y),
                    lo_f32(a.z), hi_f32(a.z), lo_f32(a.w), hi_f32(a.w)};
    for (int k = 0; k < n_peers; ++k) {
      const uint4 b = stream_load(reinterpret_cast<const uint4 *>(peers + (int64_t)k * peer_stride) + v);
      acc[0] += lo_f32(b.x); acc[1] += hi_f32(b.x); acc[2] += lo_f32(b.y); acc[3] += hi_f32(b.y);
      acc[4] += lo_f32(b.z); acc[5] += hi_f32(b.z); acc[6] += lo_f32(b.w); acc[7] += hi_f32(b.w);
    }
    if (t.res)
      drop_res8(acc, reinterpret_cast<const uint4 *>(t.res)[v], v, t.seed, t.layer, t.sb, t.thr, t.scale, t.drop);
    out[v] = make_uint4(cvt_pk(acc[0], acc[1]), cvt_pk(acc[2], acc[3]), cvt_pk(acc[4], acc[5]),
                        cvt_pk(acc[6], acc[7]));
  }
}

__global__ void __launch_bounds__(SUM_NT)
    allreduce_f32_kernel(const float4 *__restrict__ own, const float *__restrict__ peers,
                         int64_t peer_stride, int n_peers, float4 *__restrict__ out, int64_t nvec) {
  for (int64_t v = (int64_t)blockIdx.x * SUM_NT + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * SUM_NT) {
    float4 acc = own[v];
    for (int k = 0; k < n_peers; ++k) {
      const float4 b = reinterpret_cast<const float4 *>(peers + (int64_t)k * peer_stride)[v];
      acc.x += b.x; acc.y += b.y; acc.z += b.z; acc.w += b.w;
    }
    out[v] = acc;
  }
}

// ---------------------------------------------------------------------------
// Column sums, two passes with a fixed summation order (no atomics), so the
// bias gradient is bit-reproducible:
//   pass 1: partial[chunk][c] = sum of rows [64 chunk, 64 chunk + 64) of column
//           c.  A workgroup covers 256 columns x 64 rows: 8 row lanes each add
//           8 rows (16-byte loads of 8 columns), then the 8 lane sums are
//           added in lane order through LDS.
//   pass 2: db[c] = (beta ? db[c] : 0) + sum over chunks in increasing order,
//           8 chunk lanes per column, combined in lane order through LDS.
// ---------------------------------------------------------------------------
constexpr int CS_ROWS = 64;

template <bool BF16>
__global__ void __launch_bounds__(256)
    colsum_pass1(const void *__restrict__ x, int rows, int cols, int ldx, float *__restrict__ partial) {
  __shared__ float sm[8][257];
  const int cg = threadIdx.x & 31, rl = threadIdx.x >> 5;
  const int c8 = blockIdx.x * 256 + cg * 8;
  const int r0 = blockIdx.y * CS_ROWS;
  float acc[8] = {};
  if (c8 < cols) {
#pragma unroll
    for (int i = 0; i < CS_ROWS / 8; ++i) {
      const int r = r0 + rl + 8 * i;
      if (r >= rows) break;
      if constexpr (BF16) {
        const uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(x) + (int64_t)r * ldx + c8);
        acc[0] += lo_f32(a.x); acc[1] += hi_f32(a.x); acc[2] += lo_f32(a.y); acc[3] += hi_f32(a.y);
        acc[4] += lo_f32(a.z); acc[5] += hi_f32(a.z); acc[6] += lo_f32(a.w); acc[7] += hi_f32(a.w);
      } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (int64_t)r * ldx + c8);
        const float4 a = p[0], b = p[1];
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm[rl][cg * 8 + e] = acc[e];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < cols) {
    float t = sm[0][threadIdx.x];
#pragma unroll
    for (int l = 1; l < 8; ++l) t += sm[l][threadIdx.x];
    partial[(int64_t)blockIdx.y * cols + c] = t;
  }
}

__device__ __forceinline__ void colsum_pass2_body(const float *__restrict__ partial, int nchunks, int cols,
                                                  float *__restrict__ db, int beta) {
  __shared__ float sm[8][33];
  const int cl = threadIdx.x & 31, ch = threadIdx.x >> 5;
  const int c = blockIdx.x * 32 + cl;
  float t = 0.f;
  if (c < cols)
    for (int k = ch; k < nchunks; k += 8) t += partial[(int64_t)k * cols + c];
  sm[ch][cl] = t;
  __syncthreads();
  if (threadIdx.x < 32 && c < cols) {
    float r = beta ? db[c] : 0.f;
    float u = sm[0][cl];
#pragma unroll
    for (int l = 1; l < 8; ++l) u += sm[l][cl];
    db[c] = r + u;
  }
}

__global__ void __launch_bounds__(256)
    colsum_pass2(const float *__restrict__ partial, int nchunks, int cols, float *__restrict__ db, int beta) {
  colsum_pass2_body(partial, nchunks, cols, db, beta);
}

// the two column sums of the LayerNorm weight gradients in one launch:
// blockIdx.y = 0 sums partial_w into dw, 1 sums partial_b into db
__global__ void __launch_bounds__(256)
    colsum_pass2_pair(const float *__restrict__ pw, const float *__restrict__ pb, int nchunks, int cols,
                      float *__restrict__ dw, float *__restrict__ db, int beta) {
  if (blockIdx.y == 0) colsum_pass2_body(pw, nchunks, cols, dw, beta);
  else colsum_pass2_body(pb, nchunks, cols, db, beta);
}

// ---------------------------------------------------------------------------
// Full transformer block (bf16): LayerNorm forward / backward, dropout
// backward.  A row of h elements belongs to one wave (64 lanes x 16-byte
// vectors); row statistics are wave reductions in a fixed butterfly order.
// The mean and the biased variance are two passes over the row, so
// var = mean((x - mean)^2) exactly as defined.
// ---------------------------------------------------------------------------
constexpr int LN_ROWS = 4;  // rows (waves) per workgroup

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void unpack8(const uint4 a, float (&f)[8]) {
  f[0] = lo_f32(a.x); f[1] = hi_f32(a.x); f[2] = lo_f32(a.y); f[3] = hi_f32(a.y);
  f[4] = lo_f32(a.z); f[5] = hi_f32(a.z); f[6] = lo_f32(a.w); f[7] = hi_f32(a.w);
}

// mean and 1/sqrt(var + eps) of a row of hv 8-element vectors
__device__ __forceinline__ void row_stats(const uint4 *xr, int hv, int lane, float eps, float &mu, float &rstd) {
  const float inv_h = 1.f / (float)(hv * 8);
  float sum = 0.f;
  for (int j = lane; j < hv; j += 64) {
    float f[8];
    unpack8(xr[j], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += f[e];
  }
  mu = wave_sum(sum) * inv_h;
  float sq = 0.f;
  for (int j = lane; j < hv; j += 64) {
    float f[8];
    unpack8(xr[j], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dlt = f[e] - mu;
      sq += dlt * dlt;
    }
  }
  rstd = rsqrtf(wave_sum(sq) * inv_h + eps);
}

__global__ void __launch_bounds__(64 * LN_ROWS)
    ln_fwd_kernel(const uint4 *__restrict__ x, const uint4 *__restrict__ w, const uint4 *__restrict__ b,
                  uint4 *__restrict__ z, int rows, int hv, float eps) {
  const int row = blockIdx.x * LN_ROWS + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint4 *xr = x + (int64_t)row * hv;
  float mu, rstd;
  row_stats(xr, hv, lane, eps, mu, rstd);
  for (int j = lane; j < hv; j += 64) {
    float f[8], gw[8], gb[8];
    unpack8(xr[j], f);
    unpack8(w[j], gw);
    unpack8(b[j], gb);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = __builtin_fmaf((f[e] - mu) * rstd, gw[e], gb[e]);
    z[(int64_t)row * hv + j] = make_uint4(cvt_pk(f[0], f[1]), cvt_pk(f[2], f[3]), cvt_pk(f[4], f[5]),
                                          cvt_pk(f[6], f[7]));
  }
}

// The same two kernels for rows of at most 64 * RV vectors, held in
// registers: RV 16-byte vectors per lane, all of a row's loads in flight
// before the first add, so the row is read from memory once instead of once
// per pass with one load per lane in flight.  The arithmetic and its order
// are those of the kernels above (per lane in ascending vector order, then
// the wave butterfly), so the results are bit-identical to theirs.
template <int RV>
__device__ __forceinline__ void row_stats_reg(const uint4 (&xv)[RV], int hv, int lane, float eps, float &mu,
                                              float &rstd) {
  const float inv_h = 1.f / (float)(hv * 8);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < RV; ++i) {
    if (lane + 64 * i >= hv) break;
    float f[8];
    unpack8(xv[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += f[e];
  }
  mu = wave_sum(sum) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < RV; ++i) {
    if (lane + 64 * i >= hv) break;
    float f[8];
    unpack8(xv[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dlt = f[e] - mu;
      sq += dlt * dlt;
    }
  }
  rstd = rsqrtf(wave_sum(sq) * inv_h + eps);
}

template <int RV>
__device__ __forceinline__ void load_row(const uint4 *r, int hv, int lane, uint4 (&v)[RV]) {
#pragma unroll
  for (int i = 0; i < RV; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < hv ? r[j] : make_uint4(0, 0, 0, 0);
  }
}

template <int RV>
__global__ void __launch_bounds__(64 * LN_ROWS)
    ln_fwd_reg_kernel(const uint4 *__restrict__ x, const uint4 *__restrict__ w, const uint4 *__restrict__ b,
                      uint4 *__restrict__ z, int rows, int hv, float eps) {
  const int row = blockIdx.x * LN_ROWS + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  uint4 xv[RV];
  load_row<RV>(x + (int64_t)row * hv, hv, lane, xv);
  float mu, rstd;
  row_stats_reg<RV>(xv, hv, lane, eps, mu, rstd);
#pragma unroll
  for (int i = 0; i < RV; ++i) {
    const int j = lane + 64 * i;
    if (j >= hv) break;
    float f[8], gw[8], gb[8];
    unpack8(xv[i], f);
    unpack8(w[j], gw);
    unpack8(b[j], gb);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = __builtin_fmaf((f[e] - mu) * rstd, gw[e], gb[e]);
    z[(int64_t)row * hv + j] = make_uint4(cvt_pk(f[0], f[1]), cvt_pk(f[2], f[3]), cvt_pk(f[4], f[5]),
                                          cvt_pk(f[6], f[7]));
  }
}

template <int RV>
__global__ void __launch_bounds__(64 * LN_ROWS)
    ln_bwd_reg_kernel(const uint4 *__restrict__ dz, const uint4 *__restrict__ x, const uint4 *__restrict__ w,
                      const uint4 *__restrict__ g, uint4 *__restrict__ dx, float2 *__restrict__ stats, int rows,
                      int hv, float eps) {
  const int row = blockIdx.x * LN_ROWS + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t base = (int64_t)row * hv;
  uint4 xv[RV], dv[RV];
  load_row<RV>(x + base, hv, lane, xv);
  load_row<RV>(dz + base, hv, lane, dv);
  float mu, rstd;
  row_stats_reg<RV>(xv, hv, lane, eps, mu, rstd);
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < RV; ++i) {
    const int j = lane + 64 * i;
    if (j >= hv) break;
    float fx[8], fd[8], fw[8];
    unpack8(xv[i], fx);
    unpack8(dv[i], fd);
    unpack8(w[j], fw);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gy = fw[e] * fd[e];
      s1 += gy;
      s2 += gy * ((fx[e] - mu) * rstd);
    }
  }
  const float inv_h = 1.f / (float)(hv * 8);
  const float m1 = wave_sum(s1) * inv_h, m2 = wave_sum(s2) * inv_h;
#pragma unroll
  for (int i = 0; i < RV; ++i) {
    const int j = lane + 64 * i;
    if (j >= hv) break;
    float fx[8], fd[8], fw[8], fg[8], o[8];
    unpack8(xv[i], fx);
    unpack8(dv[i], fd);
    unpack8(w[j], fw);
    unpack8(g[base + j], fg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xh = (fx[e] - mu) * rstd;
      o[e] = fg[e] + rstd * (fw[e] * fd[e] - m1 - xh * m2);
    }
    dx[base + j] = make_uint4(cvt_pk(o[0], o[1]), cvt_pk(o[2], o[3]), cvt_pk(o[4], o[5]), cvt_pk(o[6], o[7]));
  }
  if (lane == 0) stats[row] = make_float2(mu, rstd);
}

// dx = g + rstd * (w dz - mean(w dz) - xhat * mean(w dz xhat)); stats[row] = (mean, rstd)
__global__ void __launch_bounds__(64 * LN_ROWS)
    ln_bwd_kernel(const uint4 *__restrict__ dz, const uint4 *__restrict__ x, const uint4 *__restrict__ w,
                  const uint4 *__restrict__ g, uint4 *__restrict__ dx, float2 *__restrict__ stats, int rows,
                  int hv, float eps) {
  const int row = blockIdx.x * LN_ROWS + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t base = (int64_t)row * hv;
  float mu, rstd;
  row_stats(x + base, hv, lane, eps, mu, rstd);
  float s1 = 0.f, s2 = 0.f;
  for (int j = lane; j < hv; j += 64) {
    float fx[8], fd[8], fw[8];
    unpack8(x[base + j], fx);
    unpack8(dz[base + j], fd);
    unpack8(w[j], fw);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gy = fw[e] * fd[e];
      s1 += gy;
      s2 += gy * ((fx[e] - mu) * rstd);
    }
  }
  const float inv_h = 1.f / (float)(hv * 8);
  const float m1 = wave_sum(s1) * inv_h, m2 = wave_sum(s2) * inv_h;
  for (int j = lane; j < hv; j += 64) {
    float fx[8], fd[8], fw[8], fg[8], o[8];
    unpack8(x[base + j], fx);
    unpack8(dz[base + j], fd);
    unpack8(w[j], fw);
    unpack8(g[base + j], fg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xh = (fx[e] - mu) * rstd;
      o[e] = fg[e] + rstd * (fw[e] * fd[e] - m1 - xh * m2);
    }
    dx[base + j] = make_uint4(cvt_pk(o[0], o[1]), cvt_pk(o[2], o[3]), cvt_pk(o[4], o[5]), cvt_pk(o[6], o[7]));
  }
  if (lane == 0) stats[row] = make_float2(mu, rstd);
}

// column partials of dw = sum_rows dz * xhat and db = sum_rows dz over chunks of
// CS_ROWS rows, in the layout and fixed order of colsum_pass1 (partial_w and
// partial_b each [chunks][h])
__global__ void __launch_bounds__(256)
    ln_grad_pass1(const bf16_t *__restrict__ dz, const bf16_t *__restrict__ x, const float2 *__restrict__ stats,
                  int rows, int h, float *__restrict__ partial_w, float *__restrict__ partial_b) {
  __shared__ float sw[8][257], sb[8][257];
  const int cg = threadIdx.x & 31, rl = threadIdx.x >> 5;
  const int c8 = blockIdx.x * 256 + cg * 8;
  const int r0 = blockIdx.y * CS_ROWS;
  float aw[8] = {}, ab[8] = {};
  if (c8 < h) {
    for (int i = 0; i < CS_ROWS / 8; ++i) {
      const int r = r0 + rl + 8 * i;
      if (r >= rows) break;
      const float2 st = stats[r];
      float fd[8], fx[8];
      unpack8(*reinterpret_cast<const uint4 *>(dz + (int64_t)r * h + c8), fd);
      unpack8(*reinterpret_cast<const uint4 *>(x + (int64_t)r * h + c8), fx);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        aw[e] += fd[e] * ((fx[e] - st.x) * st.y);
        ab[e] += fd[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sw[rl][cg * 8 + e] = aw[e];
    sb[rl][cg * 8 + e] = ab[e];
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < h) {
    float tw = sw[0][threadIdx.x], tb = sb[0][threadIdx.x];
#pragma unroll
    for (int l = 1; l < 8; ++l) {
      tw += sw[l][threadIdx.x];
      tb += sb[l][threadIdx.x];
    }
    partial_w[(int64_t)blockIdx.y * h + c] = tw;
    partial_b[(int64_t)blockIdx.y * h + c] = tb;
  }
}

__global__ void __launch_bounds__(SUM_NT)
    dropout_bwd_kernel(const uint4 *__restrict__ g, uint4 *__restrict__ out, int64_t nvec, DropRes t) {
  for (int64_t v = (int64_t)blockIdx.x * SUM_NT + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * SUM_NT) {
    float f[8];
    unpack8(g[v], f);
    if (t.drop) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint64_t c[4] = {(uint64_t)(2 * v + hh), t.sb, 0ull, 0ull};
        philox4x64(c, t.seed, t.layer);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * hh + j] = c[j] < t.thr ? f[4 * hh + j] * t.scale : 0.f;
      }
    }
    out[v] = make_uint4(cvt_pk(f[0], f[1]), cvt_pk(f[2], f[3]), cvt_pk(f[4], f[5]), cvt_pk(f[6], f[7]));
  }
}

}  // namespace

int g_sum_grid_cap = 512;  // workgroups of the AllReduce-point sum (tunable)
int g_sum_variant = 0;     // 0 automatic (per call site), 1 several vectors per thread, 2 lean

int allreduce_form(bool beside_compute) {
  if (g_sum_variant == 1) return 0;
  if (g_sum_variant == 2) return 1;
  return beside_compute ? 1 : 0;
}

hipError_t allreduce_point(bool bf16, const void *own, const void *peers, int64_t peer_stride,
                           int n_peers, void *out, int64_t n, hipStream_t s, const DropRes *tail, int form) {
  if (n <= 0) return hipSuccess;
  if (tail && tail->res && !bf16) return hipErrorInvalidValue;
  const DropRes t = tail ? *tail : DropRes{};
  const int64_t per_vec = bf16 ? 8 : 4;
  const int64_t nvec = n / per_vec;
  const int unroll = bf16 && n_peers <= 7 ? (n_peers >= 4 ? 2 : 4) : 1;
  const int64_t want = (nvec + (int64_t)SUM_NT * unroll - 1) / ((int64_t)SUM_NT * unroll);
  const dim3 grid((unsigned)(want < g_sum_grid_cap ? want : g_sum_grid_cap));
  const uint4 *o = static_cast<const uint4 *>(own);
  const bf16_t *p = static_cast<const bf16_t *>(peers);
  uint4 *y = static_cast<uint4 *>(out);
  if (!bf16) {
    OASES_LAUNCH(allreduce_f32_kernel, grid, dim3(SUM_NT), s, static_cast<const float4 *>(own),
                 static_cast<const float *>(peers), peer_stride, n_peers, static_cast<float4 *>(out), nvec);
    return hipSuccess;
  }
  if (form == 1 && n_peers <= 7) {
    // beside compute kernels: half the grid cap (measured at the 8192-hidden
    // pair: 256 workgroups leave the sums 96% hidden, 512-2048 about 90%)
    const int64_t want1 = (nvec + SUM_NT - 1) / SUM_NT, cap1 = g_sum_grid_cap < 2 ? 1 : g_sum_grid_cap / 2;
    const dim3 grid1((unsigned)(want1 < cap1 ? want1 : cap1));
    switch (n_peers) {
#define OASES_SUM_CASE(NP)                                                                                  \
  case NP:                                                                                                  \
    if (t.res) OASES_LAUNCH((allreduce_bf16_lean_kernel<NP, true>), grid1, dim3(SUM_NT), s, o, p, peer_stride, y, nvec, t); \
    else OASES_LAUNCH((allreduce_bf16_lean_kernel<NP, false>), grid1, dim3(SUM_NT), s, o, p, peer_stride, y, nvec, t); \
    break;
      OASES_SUM_CASE(0) OASES_SUM_CASE(1) OASES_SUM_CASE(2) OASES_SUM_CASE(3)
      OASES_SUM_CASE(4) OASES_SUM_CASE(5) OASES_SUM_CASE(6) OASES_SUM_CASE(7)
#undef OASES_SUM_CASE
    }
    return hipSuccess;
  }
  switch (n_peers) {
#define OASES_SUM_CASE(NP) \
  case NP: OASES_LAUNCH(allreduce_bf16_kernel<NP>, grid, dim3(SUM_NT), s, o, p, peer_stride, y, nvec, t); break;
    OASES_SUM_CASE(0) OASES_SUM_CASE(1) OASES_SUM_CASE(2) OASES_SUM_CASE(3)
    OASES_SUM_CASE(4) OASES_SUM_CASE(5) OASES_SUM_CASE(6) OASES_SUM_CASE(7)
#undef OASES_SUM_CASE
    default:
      OASES_LAUNCH(allreduce_bf16_many_kernel, grid, dim3(SUM_NT), s, o, p, peer_stride, n_peers, y, nvec, t);
  }
  return hipSuccess;
}

void allreduce_set_grid_cap(int cap) { g_sum_grid_cap = cap; }
void allreduce_set_variant(int v) { g_sum_variant = v; }

int allreduce_fused_wgs(int64_t nvec) {
  // half the standalone grid cap: beside a GEMM's tiles, a larger sum grid
  // takes CUs the GEMM needs (measured best at 128-256 workgroups)
  const int64_t want = (nvec + 256 * 2 - 1) / (256 * 2);
  const int64_t cap = g_sum_grid_cap < 16 ? 8 : g_sum_grid_cap / 2;
  const int64_t w = want < cap ? want : cap;
  return (int)((w + 7) / 8 * 8);
}

hipError_t layer_norm_fwd(const void *x, const void *w, const void *b, void *z, int rows, int h, float eps,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + LN_ROWS - 1) / LN_ROWS), block(64 * LN_ROWS);
  const uint4 *xp = static_cast<const uint4 *>(x), *wp = static_cast<const uint4 *>(w),
              *bp = static_cast<const uint4 *>(b);
  uint4 *zp = static_cast<uint4 *>(z);
  const int hv = h / 8;
  // rows held in registers up to 64 x 16 vectors (h = 8192); longer rows in passes
  if (hv <= 64 * 4) OASES_LAUNCH(ln_fwd_reg_kernel<4>, grid, block, s, xp, wp, bp, zp, rows, hv, eps);
  else if (hv <= 64 * 8) OASES_LAUNCH(ln_fwd_reg_kernel<8>, grid, block, s, xp, wp, bp, zp, rows, hv, eps);
  else if (hv <= 64 * 16) OASES_LAUNCH(ln_fwd_reg_kernel<16>, grid, block, s, xp, wp, bp, zp, rows, hv, eps);
  else OASES_LAUNCH(ln_fwd_kernel, grid, block, s, xp, wp, bp, zp, rows, hv, eps);
  return hipGetLastError();
}

int64_t layer_norm_partial_floats(int rows, int h) {
  return 2 * (int64_t)((rows + CS_ROWS - 1) / CS_ROWS) * h;
}

hipError_t layer_norm_bwd(const void *dz, const void *x, const void *w, const void *g, void *dx, float *stats,
                          float *partial, int rows, int h, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  {
    const dim3 grid((rows + LN_ROWS - 1) / LN_ROWS), block(64 * LN_ROWS);
    const uint4 *dzp = static_cast<const uint4 *>(dz), *xp = static_cast<const uint4 *>(x),
                *wp = static_cast<const uint4 *>(w), *gp = static_cast<const uint4 *>(g);
    uint4 *dxp = static_cast<uint4 *>(dx);
    float2 *st = reinterpret_cast<float2 *>(stats);
    const int hv = h / 8;
    if (hv <= 64 * 4)
      OASES_LAUNCH(ln_bwd_reg_kernel<4>, grid, block, s, dzp, xp, wp, gp, dxp, st, rows, hv, eps);
    else if (hv <= 64 * 8)
      OASES_LAUNCH(ln_bwd_reg_kernel<8>, grid, block, s, dzp, xp, wp, gp, dxp, st, rows, hv, eps);
    else if (hv <= 64 * 16)
      OASES_LAUNCH(ln_bwd_reg_kernel<16>, grid, block, s, dzp, xp, wp, gp, dxp, st, rows, hv, eps);
    else
      OASES_LAUNCH(ln_bwd_kernel, grid, block, s, dzp, xp, wp, gp, dxp, st, rows, hv, eps);
  }
  const int nchunks = (rows + CS_ROWS - 1) / CS_ROWS;
  float *pw = partial, *pb = partial + (int64_t)nchunks * h;
  OASES_LAUNCH(ln_grad_pass1, dim3((h + 255) / 256, nchunks), dim3(256), s, static_cast<const bf16_t *>(dz),
               static_cast<const bf16_t *>(x), reinterpret_cast<const float2 *>(stats), rows, h, pw, pb);
  return hipGetLastError();
}

hipError_t layer_norm_wgrad(const float *partial, float *dw, float *db, int rows, int h, int beta,
                            hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int nchunks = (rows + CS_ROWS - 1) / CS_ROWS;
  const float *pw = partial, *pb = partial + (int64_t)nchunks * h;
  OASES_LAUNCH(colsum_pass2_pair, dim3((h + 31) / 32, 2), dim3(256), s, pw, pb, nchunks, h, dw, db, beta);
  return hipGetLastError();
}

hipError_t dropout_bwd(const void *g, void *out, int64_t n, const DropRes &t, hipStream_t s) {
  const int64_t nvec = n / 8;
  if (nvec <= 0) return hipSuccess;
  const int64_t want = (nvec + SUM_NT - 1) / SUM_NT;
  OASES_LAUNCH(dropout_bwd_kernel, dim3((unsigned)(want < 1024 ? want : 1024)), dim3(SUM_NT), s,
               static_cast<const uint4 *>(g), static_cast<uint4 *>(out), nvec, t);
  return hipGetLastError();
}

int64_t colsum_partial_floats(int rows, int cols) {
  return (int64_t)((rows + CS_ROWS - 1) / CS_ROWS) * cols;
}

hipError_t colsum(bool bf16, const void *x, int rows, int cols, int ldx, float *partial, float *db,
                  int beta, hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  const int nchunks = (rows + CS_ROWS - 1) / CS_ROWS;
  if (nchunks > 0) {
    dim3 g1((cols + 255) / 256, nchunks);
    if (bf16)
      OASES_LAUNCH(colsum_pass1<true>, g1, dim3(256), s, x, rows, cols, ldx, partial);
    else
      OASES_LAUNCH(colsum_pass1<false>, g1, dim3(256), s, x, rows, cols, ldx, partial);
  }
  OASES_LAUNCH(colsum_pass2, dim3((cols + 31) / 32), dim3(256), s, partial, nchunks, cols, db,
                     beta);
  return hipGetLastError();
}

}  // namespace oases
