// Causal multi-head attention of the attention block's shard (bf16, MFMA).
//
// QKV is [nb*s, 3a] with columns [Q | K | V], each head-major (head h owns
// columns h*d .. h*d+d-1 of its part); O is [nb*s, a].  Per (sequence, head):
//   O = softmax(Q K^T / sqrt(d) + causal mask) V,   lse = log-sum-exp of a row.
// lse and delta are stored per (sequence, head) with a row stride of
// s_pad = s rounded up to 64, so a 64-row block never reads past its row.
//
// All kernels walk 64-row blocks of the "other" operand through an LDS ring
// fed by the gfx950 LDS DMA, STAGES-1 blocks ahead (the same scheme as the
// GEMM).  A block that an MFMA reads with d as the reduction index is stored
// k-contiguous ("KC": [64][64] slabs, 16-byte chunks swizzled by row); a block
// that an MFMA reads with the row index as the reduction ("MC", e.g. V in
// O^T += V^T P^T) is stored as-is and read with the transposing LDS read
// ds_read_b64_tr_b16.  Accumulator tiles are arranged so that a lane owns one
// query (forward, dQ) or one key (dK/dV): the online-softmax row statistics
// are per-lane values plus one exchange with the lane 32 away, and the P / dS
// tile in accumulator layout is directly the B operand of the next MFMA once
// the A operand is read with the same (accumulator-row) order of its k index.
//
// Backward (no atomics): delta = rowsum(dO * O); the dK/dV kernel owns keys
// and walks query blocks (S = Q K^T, dP = dO V^T, dV^T += dO^T P,
// dK^T += Q^T dS); the dQ kernel owns queries and walks key blocks
// (S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T).  P is rebuilt from lse.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

constexpr int BLK = 64;  // rows per staged block
constexpr float LOG2E = 1.4426950408889634f;

using C0 = std::integral_constant<int, 0>;
using C1 = std::integral_constant<int, 1>;
using C2 = std::integral_constant<int, 2>;

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_frag(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 load_frag(const bf16_t *p) {
  return as_frag(*reinterpret_cast<const uint4 *>(p));
}
__device__ __forceinline__ void zero(f32x16 &a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.f;
}
// accumulator registers [8h, 8h+8) -> bf16 B-operand fragment
__device__ __forceinline__ bf16x8 acc_to_frag(const f32x16 &a, int h) {
  return as_frag(make_uint4(pack_bf16x2(a[8 * h + 0], a[8 * h + 1]), pack_bf16x2(a[8 * h + 2], a[8 * h + 3]),
                            pack_bf16x2(a[8 * h + 4], a[8 * h + 5]), pack_bf16x2(a[8 * h + 6], a[8 * h + 7])));
}
// row (within a 32-row MFMA tile) held in accumulator register r by lane half hl
__device__ __forceinline__ int acc_row(int r, int hl) { return (r >> 2) * 8 + hl * 4 + (r & 3); }

// Make the compiler wait for (and keep) register values loaded from global
// memory before DMA is issued: DMA is invisible to its wait counting, so a
// first use later on would otherwise wait for all outstanding DMA too.
__device__ __forceinline__ void settle(const bf16x8 &v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  asm volatile("" ::"v"(u));
}
__device__ __forceinline__ void settle(float v) { asm volatile("" ::"v"(v)); }

// ---- block tiles -------------------------------------------------------------

// KC block: 64 rows x D, as D/64 slabs of [64][64] with chunk c of row r at
// c ^ ((r ^ (r >> 3)) & 7).  Unit u (1 KB) = 8 rows of one slab.
template <int D>
struct KcBlock {
  static constexpr int UNITS = D / 8;
  __device__ __forceinline__ static int key(int r) { return (r ^ (r >> 3)) & 7; }
  __device__ __forceinline__ static void dma(const bf16_t *g, int ld, int row0, int nvalid, int u,
                                             bf16_t *tile, int lane) {
    const int slab = u >> 3, rb = u & 7;
    const int r = rb * 8 + (lane >> 3);
    const int c = (lane & 7) ^ key(r);
    const bool ok = row0 + r < nvalid;
    dma16(ok ? g + (int64_t)(row0 + r) * ld + slab * 64 + c * 8 : zero_page(), tile + slab * 4096 + rb * 512);
  }
  // 8 consecutive d (half hl of 16-wide substep kk) of block row `row`
  __device__ __forceinline__ static bf16x8 frag(const bf16_t *tile, int row, int kk, int hl) {
    const int slab = kk >> 2, c = ((kk & 3) << 1) + hl;
    return load_frag(tile + slab * 4096 + row * 64 + ((c ^ key(row)) << 3));
  }
};

// MC block: 64 rows x D stored as-is, 16-byte chunk c of row k at c ^ mc_swz(k).
// Unit u (1 KB) = 1024 / (2 D) rows.
template <int D>
struct McBlock {
  static constexpr int UNITS = D / 8;
  __device__ __forceinline__ static void dma(const bf16_t *g, int ld, int row0, int nvalid, int u,
                                             bf16_t *tile, int lane) {
    const int byte = u * 1024 + lane * 16;
    const int kr = byte / (2 * D), cp = (byte % (2 * D)) >> 4;
    const int c = cp ^ mc_swz<D>(kr);
    const bool ok = row0 + kr < nvalid;
    dma16(ok ? g + (int64_t)(row0 + kr) * ld + c * 8 : zero_page(), tile + u * 512);
  }
  // Transposed fragment: column `col` (0..D-1) of the block at the 8 rows
  // {k_lo + hl*4 + 0..3, k_hi + hl*4 + 0..3}, the accumulator-row order of
  // 16 rows starting at k_lo (k_hi = k_lo + 8).  In each 16-lane group,
  // source lane s addresses row base + s/4 at columns col0 + 4 (s % 4); the
  // transposing read then hands lane i rows base..base+3 of column col0 + i.
  __device__ __forceinline__ static bf16x8 frag_t(const bf16_t *tile, int col, int k_lo, int hl) {
    const int s = threadIdx.x & 15;
    const int n = (col - s) + 4 * (s & 3);
    v4i16 v[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = k_lo + r * 8 + hl * 4 + (s >> 2);
      const bf16_t *a = tile + k * D + (((n >> 3) ^ mc_swz<D>(k)) << 3) + (n & 7);
      v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(lds_void_t *)a);
    }
    const uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
    return as_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
};

// Walk blocks 0..nblk-1 through a ring of STAGES LDS slots (static slot
// indices, so the compiler sees distinct LDS objects).  issue(slot, j) starts
// the DMA of block j (exactly DL DMA instructions per wave); compute(slot, j)
// consumes it.  Block j's DMA is awaited with a counted vmcnt wait.
template <int STAGES, int DL, bool MULTI, class Issue, class Compute>
__device__ __forceinline__ void pipeline(int nblk, Issue &&issue, Compute &&compute) {
  static_assert(STAGES == 2 || STAGES == 3, "2 or 3 stages");
  if (nblk <= 0) return;
  issue(C0{}, 0);
  if constexpr (STAGES == 3)
    if (nblk > 1) issue(C1{}, 1);
  auto step = [&](auto I, int j) {
    using AHEAD = std::integral_constant<int, (decltype(I)::value + STAGES - 1) % STAGES>;
    if constexpr (STAGES == 3) {
      if (j + 1 < nblk) wait_vmcnt<DL>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    if constexpr (MULTI) lds_barrier();
    if (j + STAGES - 1 < nblk) issue(AHEAD{}, j + STAGES - 1);
    compute(I, j);
  };
  int j = 0;
  for (; j + STAGES <= nblk; j += STAGES) {
    step(C0{}, j);
    step(C1{}, j + 1);
    if constexpr (STAGES == 3) step(C2{}, j + 2);
  }
  if (j < nblk) step(C0{}, j);
  if constexpr (STAGES == 3)
    if (j + 1 < nblk) step(C1{}, j + 1);
}

// Work split (all kernels): a workgroup owns one 32-row tile (queries for the
// forward and dQ, keys for dK/dV) and walks the other dimension in steps of
// BPS 64-row blocks, staged cooperatively.  Its NW = 2 BPS waves each take a
// 32-row slice of every step (block w / 2, half w % 2), so all waves work on
// the same tile; their partial results are combined through LDS in wave order
// at the end (a fixed order: results are deterministic).

template <int D>
struct Split {
  static constexpr int BPS = D == 64 ? 2 : 1;  // 64-row blocks per step
  static constexpr int NW = 2 * BPS;           // waves per workgroup
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, int STAGES>
__global__ void __launch_bounds__(64 * Split<D>::NW)
    attn_fwd_kernel(const bf16_t *__restrict__ qkv, bf16_t *__restrict__ out, float *__restrict__ lse,
                    int s, int s_pad, int nh, int causal, float scale_log2) {
  constexpr int BPS = Split<D>::BPS, NW = Split<D>::NW, TE = BLK * D, ST = BPS * TE;
  constexpr int U = BPS * (KcBlock<D>::UNITS + McBlock<D>::UNITS);
  static_assert(U % NW == 0, "units per wave");
  constexpr int DL = U / NW;
  // LDS arena: K slots [0, STAGES), V slots [STAGES, 2 STAGES); reused for the reduction
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * STAGES * ST];
  static_assert((NW * D * 32 + NW * 64) * 2 <= 2 * STAGES * ST, "reduction fits the arena");
  auto kslot = [&](auto I) { return smem + decltype(I)::value * ST; };
  auto vslot = [&](auto I) { return smem + (STAGES + decltype(I)::value) * ST; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wb = wave >> 1, wsub = wave & 1;  // this wave's block of a step and half of it
  const int ntile = (s + 31) / 32;
  const int q0 = (ntile - 1 - (int)blockIdx.x) * 32;  // heaviest causal tiles first
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const int qi = q0 + l32;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qi < s ? load_frag(Qp + (int64_t)qi * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    settle(qf[kk]);
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(oacc[t]);
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = causal ? min(s, q0 + 32) : s;
  const int nkb = (kend + BLK - 1) / BLK;
  auto issue = [&](auto I, int j) {
    bf16_t *k_s = kslot(I), *v_s = vslot(I);
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const int u = i * NW + wave;
      constexpr int PB = KcBlock<D>::UNITS + McBlock<D>::UNITS;  // units per block
      const int blk = u / PB, v = u % PB;
      const int key0 = (j * BPS + blk) * BLK;
      if (v < KcBlock<D>::UNITS) KcBlock<D>::dma(Kp, ld, key0, s, v, k_s + blk * TE, lane);
      else McBlock<D>::dma(Vp, ld, key0, s, v - KcBlock<D>::UNITS, v_s + blk * TE, lane);
    }
  };
  auto compute = [&](auto I, int j) {
    const int kb = j * BPS + wb;
    const int k0 = kb * BLK + wsub * 32;  // this wave's 32 keys
    if (kb >= nkb || k0 >= s || (causal && k0 > q0 + 31)) return;
    const bf16_t *k_s = kslot(I) + wb * TE;
    const bf16_t *v_s = vslot(I) + wb * TE;
    f32x16 st;
    zero(st);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      st = mfma32(KcBlock<D>::frag(k_s, wsub * 32 + l32, kk, hl), qf[kk], st);
    // st[r] = S^T[key][q]: key = k0 + acc_row(r, hl), q = qi
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + acc_row(r, hl);
      float x = st[r] * scale_log2;
      if (key >= s || (causal && key > qi)) x = -INFINITY;
      st[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - base);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2f(st[r] - base);
      st[r] = p;
      rs += p;
    }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 pf = acc_to_frag(st, hh);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        oacc[t] = mfma32(McBlock<D>::frag_t(v_s, t * 32 + l32, wsub * 32 + hh * 16, hl), pf, oacc[t]);
    }
  };
  pipeline<STAGES, DL, true>((nkb + BPS - 1) / BPS, issue, compute);

  // combine the waves' (m, l, O) in wave order: O = sum_w 2^(m_w - m) O_w / sum_w 2^(m_w - m) l_w
  lds_barrier();
  float *red = reinterpret_cast<float *>(smem);  // NW x [D][32] partial O
  float *ml = red + NW * D * 32;                  // [NW][2][32] m and l
  if (hl == 0) {
    ml[(wave * 2 + 0) * 32 + l32] = m_run;
    ml[(wave * 2 + 1) * 32 + l32] = l_run;
  }
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * D + t * 32 + acc_row(r, hl)) * 32 + l32] = oacc[t][r];
  lds_barrier();
  // thread -> (query q, 8 consecutive d): 32 queries x D/8 chunks over 64*NW threads
  for (int c = threadIdx.x; c < 32 * (D / 8); c += 64 * NW) {
    const int q = c % 32, d0 = (c / 32) * 8;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, ml[(w * 2) * 32 + q]);
    const float base = m == -INFINITY ? 0.f : m;
    float f[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = exp2f(ml[(w * 2) * 32 + q] - base);
      L += f[w] * ml[(w * 2 + 1) * 32 + q];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += f[w] * red[(w * D + d0 + e) * 32 + q];
      o[e] = acc * inv;
    }
    const int qq = q0 + q;
    if (qq < s) {
      *reinterpret_cast<uint4 *>(out + (int64_t)(b * s + qq) * a + h * D + d0) =
          make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                     pack_bf16x2(o[6], o[7]));
      if (d0 == 0) lse[(int64_t)bh * s_pad + qq] = (base + log2f(L)) * 0.69314718055994531f;
    }
  }
}

// ---------------------------------------------------------------------------
// backward: delta = rowsum(dO * O) per (sequence, head, query)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
    attn_delta_kernel(const bf16_t *__restrict__ o, const bf16_t *__restrict__ dout,
                      float *__restrict__ delta, int nb, int s, int s_pad, int nh) {
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
  delta[((int64_t)b * nh + h) * s_pad + t] = acc;
}

// sum the waves' [D][32] float partials (in wave order) and store them as bf16
// rows of dst (row r of the tile at dst + r*ld), times `scale`
template <int D, int NW>
__device__ __forceinline__ void reduce_store(const float *red, bf16_t *dst, int ld, int row0, int nrows,
                                             float scale) {
  for (int c = threadIdx.x; c < 32 * (D / 8); c += 64 * NW) {
    const int q = c % 32, d0 = (c / 32) * 8;
    if (row0 + q >= nrows) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += red[(w * D + d0 + e) * 32 + q];
      o[e] = acc * scale;
    }
    *reinterpret_cast<uint4 *>(dst + (int64_t)(row0 + q) * ld + d0) =
        make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                   pack_bf16x2(o[6], o[7]));
  }
}

// write a wave's [D x 32] accumulator tiles (rows d, columns = the tile's rows) to red[wave]
template <int D>
__device__ __forceinline__ void stash(float *red, int wave, const f32x16 (&acc)[D / 32], int l32, int hl) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * D + t * 32 + acc_row(r, hl)) * 32 + l32] = acc[t][r];
}

// ---------------------------------------------------------------------------
// backward: dK, dV.  The workgroup owns 32 keys; query blocks of Q and dO are
// staged both KC (for S and dP) and MC (for the transposed reads of dV, dK).
// ---------------------------------------------------------------------------
template <int D, int STAGES>
__global__ void __launch_bounds__(64 * Split<D>::NW)
    attn_bwd_dkdv_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                         const float *__restrict__ lse, const float *__restrict__ delta,
                         bf16_t *__restrict__ dqkv, int s, int s_pad, int nh, int causal,
                         float scale_log2, float scale) {
  constexpr int BPS = Split<D>::BPS, NW = Split<D>::NW, TE = BLK * D, ST = BPS * TE;
  constexpr int PB = 4 * (D / 8);  // tile units per block (Q, dO, each KC and MC)
  static_assert((BPS * PB) % NW == 0, "units per wave");
  constexpr int DL = BPS * PB / NW + 1;  // + this wave's lse/delta unit
  // LDS arena: slot i of tile kind t (Q KC, Q MC, dO KC, dO MC) at (t * STAGES + i) * ST,
  // then per-slot lse/delta; the tile part is reused for the reduction
  __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * STAGES * ST];
  __shared__ __attribute__((aligned(1024))) float sL[STAGES * NW * 256];
  static_assert(NW * D * 32 * 2 <= 4 * STAGES * ST, "reduction fits the arena");
  auto slot = [&](int t, auto I) { return smem + (t * STAGES + decltype(I)::value) * ST; };
  auto lslot = [&](auto I) { return sL + decltype(I)::value * NW * 256; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wb = wave >> 1, wsub = wave & 1;
  const int k0 = blockIdx.x * 32;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const float *lp = lse + (int64_t)bh * s_pad, *dp = delta + (int64_t)bh * s_pad;
  const int kj = k0 + l32;

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bool ok = kj < s;
    kf[kk] = ok ? load_frag(Kp + (int64_t)kj * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    vf[kk] = ok ? load_frag(Vp + (int64_t)kj * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    settle(kf[kk]);
    settle(vf[kk]);
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) { zero(dv[t]); zero(dk[t]); }

  const int qstart = causal ? k0 / BLK : 0;  // first query block that sees these keys
  const int nqb = (s + BLK - 1) / BLK;
  auto slice_q0 = [&](int j) { return (qstart + j * BPS + wb) * BLK + wsub * 32; };
  auto issue = [&](auto I, int j) {
    bf16_t *qk = slot(0, I), *qm = slot(1, I), *ok_ = slot(2, I), *om = slot(3, I);
#pragma unroll
    for (int i = 0; i < DL - 1; ++i) {
      const int u = i * NW + wave;
      const int blk = u / PB, t = (u % PB) / (D / 8), v = u % (D / 8);
      const int q0b = (qstart + j * BPS + blk) * BLK;
      if (t == 0) KcBlock<D>::dma(Qp, ld, q0b, s, v, qk + blk * TE, lane);
      else if (t == 1) McBlock<D>::dma(Qp, ld, q0b, s, v, qm + blk * TE, lane);
      else if (t == 2) KcBlock<D>::dma(dOp, a, q0b, s, v, ok_ + blk * TE, lane);
      else McBlock<D>::dma(dOp, a, q0b, s, v, om + blk * TE, lane);
    }
    // lse / delta of this wave's 32 queries: lanes 0-7 lse, lanes 8-15 delta
    float *ldst = lslot(I) + wave * 256;
    const int qs = slice_q0(j);
    const bool inb = qs < s_pad;  // slice rows exist in the padded arrays
    const float *src = !inb ? nullptr : (lane < 8 ? lp + qs + lane * 4 : (lane < 16 ? dp + qs + (lane - 8) * 4 : nullptr));
    dma16(src ? reinterpret_cast<const bf16_t *>(src) : zero_page(), reinterpret_cast<bf16_t *>(ldst));
  };
  auto compute = [&](auto I, int j) {
    const int qb = qstart + j * BPS + wb;
    const int qs = slice_q0(j);  // this wave's 32 queries
    if (qb >= nqb || qs >= s || (causal && k0 > qs + 31)) return;
    const bf16_t *qk = slot(0, I) + wb * TE, *qm = slot(1, I) + wb * TE;
    const bf16_t *ok_ = slot(2, I) + wb * TE, *om = slot(3, I) + wb * TE;
    const float *ls = lslot(I) + wave * 256;
    f32x16 sacc, dpacc;
    zero(sacc);
    zero(dpacc);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      sacc = mfma32(KcBlock<D>::frag(qk, wsub * 32 + l32, kk, hl), kf[kk], sacc);
      dpacc = mfma32(KcBlock<D>::frag(ok_, wsub * 32 + l32, kk, hl), vf[kk], dpacc);
    }
    // sacc[r]: S[q][key], q = qs + acc_row(r, hl), key = kj
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int ql0 = g4 * 8 + hl * 4;  // 4 consecutive queries of the slice
      const float4 L4 = *reinterpret_cast<const float4 *>(ls + ql0);
      const float4 D4 = *reinterpret_cast<const float4 *>(ls + 32 + ql0);
      const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = g4 * 4 + e, q = qs + ql0 + e;
        float p = exp2f(sacc[r] * scale_log2 - Lv[e] * LOG2E);
        if (q >= s || (causal && kj > q)) p = 0.f;
        sacc[r] = p;
        dpacc[r] = p * (dpacc[r] - Dv[e]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 pfr = acc_to_frag(sacc, hh), dsf = acc_to_frag(dpacc, hh);
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        dv[t] = mfma32(McBlock<D>::frag_t(om, t * 32 + l32, wsub * 32 + hh * 16, hl), pfr, dv[t]);
        dk[t] = mfma32(McBlock<D>::frag_t(qm, t * 32 + l32, wsub * 32 + hh * 16, hl), dsf, dk[t]);
      }
    }
  };
  pipeline<STAGES, DL, true>((nqb - qstart + BPS - 1) / BPS, issue, compute);

  lds_barrier();
  float *red = reinterpret_cast<float *>(smem);  // NW x [D][32]
  stash<D>(red, wave, dk, l32, hl);
  lds_barrier();
  reduce_store<D, NW>(red, dqkv + (int64_t)b * s * ld + a + h * D, ld, k0, s, scale);
  lds_barrier();
  stash<D>(red, wave, dv, l32, hl);
  lds_barrier();
  reduce_store<D, NW>(red, dqkv + (int64_t)b * s * ld + 2 * a + h * D, ld, k0, s, 1.f);
}

// ---------------------------------------------------------------------------
// backward: dQ.  The workgroup owns 32 queries; key blocks of K (KC and MC)
// and V (KC) are staged.
// ---------------------------------------------------------------------------
template <int D, int STAGES>
__global__ void __launch_bounds__(64 * Split<D>::NW)
    attn_bwd_dq_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                       const float *__restrict__ lse, const float *__restrict__ delta,
                       bf16_t *__restrict__ dqkv, int s, int s_pad, int nh, int causal,
                       float scale_log2, float scale) {
  constexpr int BPS = Split<D>::BPS, NW = Split<D>::NW, TE = BLK * D, ST = BPS * TE;
  constexpr int PB = 3 * (D / 8);
  static_assert((BPS * PB) % NW == 0, "units per wave");
  constexpr int DL = BPS * PB / NW;
  // LDS arena: slot i of tile kind t (K KC, K MC, V KC) at (t * STAGES + i) * ST
  __shared__ __attribute__((aligned(1024))) bf16_t smem[3 * STAGES * ST];
  static_assert(NW * D * 32 * 2 <= 3 * STAGES * ST, "reduction fits the arena");
  auto slot = [&](int t, auto I) { return smem + (t * STAGES + decltype(I)::value) * ST; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wb = wave >> 1, wsub = wave & 1;
  const int ntile = (s + 31) / 32;
  const int q0 = (ntile - 1 - (int)blockIdx.x) * 32;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const int qi = q0 + l32;
  const bool qok = qi < s;

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qok ? load_frag(Qp + (int64_t)qi * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    df[kk] = qok ? load_frag(dOp + (int64_t)qi * a + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    settle(qf[kk]);
    settle(df[kk]);
  }
  const float lq = qok ? lse[(int64_t)bh * s_pad + qi] * LOG2E : 0.f;
  const float dlt = qok ? delta[(int64_t)bh * s_pad + qi] : 0.f;
  settle(lq);
  settle(dlt);
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(dq[t]);

  const int kend = causal ? min(s, q0 + 32) : s;
  const int nkb = (kend + BLK - 1) / BLK;
  auto issue = [&](auto I, int j) {
    bf16_t *kk_ = slot(0, I), *km = slot(1, I), *vk = slot(2, I);
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const int u = i * NW + wave;
      const int blk = u / PB, t = (u % PB) / (D / 8), v = u % (D / 8);
      const int key0 = (j * BPS + blk) * BLK;
      if (t == 0) KcBlock<D>::dma(Kp, ld, key0, s, v, kk_ + blk * TE, lane);
      else if (t == 1) McBlock<D>::dma(Kp, ld, key0, s, v, km + blk * TE, lane);
      else KcBlock<D>::dma(Vp, ld, key0, s, v, vk + blk * TE, lane);
    }
  };
  auto compute = [&](auto I, int j) {
    const int kb = j * BPS + wb;
    const int kb0 = kb * BLK + wsub * 32;  // this wave's 32 keys
    if (kb >= nkb || kb0 >= s || q0 >= s || (causal && kb0 > q0 + 31)) return;
    const bf16_t *kk_ = slot(0, I) + wb * TE, *km = slot(1, I) + wb * TE;
    const bf16_t *vk = slot(2, I) + wb * TE;
    f32x16 sacc, dpacc;
    zero(sacc);
    zero(dpacc);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      sacc = mfma32(KcBlock<D>::frag(kk_, wsub * 32 + l32, kk, hl), qf[kk], sacc);
      dpacc = mfma32(KcBlock<D>::frag(vk, wsub * 32 + l32, kk, hl), df[kk], dpacc);
    }
    // sacc[r]: S^T[key][q], key = kb0 + acc_row(r, hl), q = qi
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb0 + acc_row(r, hl);
      float p = exp2f(sacc[r] * scale_log2 - lq);
      if (!qok || key >= s || (causal && key > qi)) p = 0.f;
      dpacc[r] = p * (dpacc[r] - dlt);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 dsf = acc_to_frag(dpacc, hh);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        dq[t] = mfma32(McBlock<D>::frag_t(km, t * 32 + l32, wsub * 32 + hh * 16, hl), dsf, dq[t]);
    }
  };
  pipeline<STAGES, DL, true>((nkb + BPS - 1) / BPS, issue, compute);

  lds_barrier();
  float *red = reinterpret_cast<float *>(smem);  // NW x [D][32]
  stash<D>(red, wave, dq, l32, hl);
  lds_barrier();
  reduce_store<D, NW>(red, dqkv + (int64_t)b * s * ld + h * D, ld, q0, s, scale);
}

// ---------------------------------------------------------------------------
// Query-parallel variant for long sequences: a workgroup owns 128 rows
// (4 waves x 32) and every staged 64-row block of the other operand is shared
// by the 4 waves, which cuts the K/V (Q/dO) re-reads by 4x compared with the
// split variant.  Same tiles, pipeline and MFMA arrangement.
// ---------------------------------------------------------------------------
constexpr int QP_NW = 4;

template <int D, int STAGES>
__global__ void __launch_bounds__(64 * QP_NW)
    attn_fwd_qp_kernel(const bf16_t *__restrict__ qkv, bf16_t *__restrict__ out, float *__restrict__ lse,
                       int s, int s_pad, int nh, int causal, float scale_log2) {
  constexpr int NW = QP_NW, QT = 32 * NW, TE = BLK * D;
  constexpr int U = KcBlock<D>::UNITS + McBlock<D>::UNITS;
  static_assert(U % NW == 0, "units per wave");
  constexpr int DL = U / NW;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * STAGES * TE];
  auto kslot = [&](auto I) { return smem + decltype(I)::value * TE; };
  auto vslot = [&](auto I) { return smem + (STAGES + decltype(I)::value) * TE; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int ntile = (s + QT - 1) / QT;
  const int q0 = (ntile - 1 - (int)blockIdx.x) * QT;  // heaviest causal tiles first
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const int qw = q0 + wave * 32, qi = qw + l32;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qi < s ? load_frag(Qp + (int64_t)qi * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    settle(qf[kk]);
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(oacc[t]);
  float m_run = -INFINITY, l_run = 0.f;

  auto issue = [&](auto I, int j) {
    bf16_t *k_s = kslot(I), *v_s = vslot(I);
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const int u = i * NW + wave;
      if (u < KcBlock<D>::UNITS) KcBlock<D>::dma(Kp, ld, j * BLK, s, u, k_s, lane);
      else McBlock<D>::dma(Vp, ld, j * BLK, s, u - KcBlock<D>::UNITS, v_s, lane);
    }
  };
  auto compute = [&](auto I, int j) {
    const int kb0 = j * BLK;
    if (qw >= s || (causal && kb0 > qw + 31)) return;
    const bf16_t *k_s = kslot(I), *v_s = vslot(I);
    f32x16 st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      zero(st[sub]);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        st[sub] = mfma32(KcBlock<D>::frag(k_s, sub * 32 + l32, kk, hl), qf[kk], st[sub]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + sub * 32 + acc_row(r, hl);
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
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 pf = acc_to_frag(st[c >> 1], c & 1);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        oacc[t] = mfma32(McBlock<D>::frag_t(v_s, t * 32 + l32, c * 16, hl), pf, oacc[t]);
    }
  };
  const int kend = causal ? min(s, q0 + QT) : s;
  pipeline<STAGES, DL, true>((kend + BLK - 1) / BLK, issue, compute);

  if (qi < s) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16_t *op = out + (int64_t)(b * s + qi) * a + h * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = t * 32 + jj * 8 + hl * 4;
        *reinterpret_cast<uint2 *>(op + d0) =
            make_uint2(pack_bf16x2(oacc[t][jj * 4 + 0] * inv, oacc[t][jj * 4 + 1] * inv),
                       pack_bf16x2(oacc[t][jj * 4 + 2] * inv, oacc[t][jj * 4 + 3] * inv));
      }
    if (hl == 0) lse[(int64_t)bh * s_pad + qi] = (m_run + log2f(l_run)) * 0.69314718055994531f;
  }
}

template <int D, int STAGES>
__global__ void __launch_bounds__(64 * QP_NW)
    attn_bwd_dkdv_qp_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                            const float *__restrict__ lse, const float *__restrict__ delta,
                            bf16_t *__restrict__ dqkv, int s, int s_pad, int nh, int causal,
                            float scale_log2, float scale) {
  constexpr int NW = QP_NW, KT = 32 * NW, TE = BLK * D, QPW = BLK / NW;
  constexpr int UT = 4 * (D / 8);
  static_assert(UT % NW == 0, "units per wave");
  constexpr int DL = UT / NW + 1;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * STAGES * TE];
  __shared__ __attribute__((aligned(1024))) float sL[STAGES * NW * 256];
  auto slot = [&](int t, auto I) { return smem + (t * STAGES + decltype(I)::value) * TE; };
  auto lslot = [&](auto I) { return sL + decltype(I)::value * NW * 256; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int k0 = blockIdx.x * KT;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const float *lp = lse + (int64_t)bh * s_pad, *dp = delta + (int64_t)bh * s_pad;
  const int kw = k0 + wave * 32, kj = kw + l32;

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bool ok = kj < s;
    kf[kk] = ok ? load_frag(Kp + (int64_t)kj * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    vf[kk] = ok ? load_frag(Vp + (int64_t)kj * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    settle(kf[kk]);
    settle(vf[kk]);
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) { zero(dv[t]); zero(dk[t]); }

  const int qstart = causal ? k0 / BLK : 0;
  auto issue = [&](auto I, int jj) {
    const int q0b = (jj + qstart) * BLK;
    bf16_t *qk = slot(0, I), *qm = slot(1, I), *ok_ = slot(2, I), *om = slot(3, I);
#pragma unroll
    for (int i = 0; i < UT / NW; ++i) {
      const int u = i * NW + wave, t = u / (D / 8), v = u % (D / 8);
      if (t == 0) KcBlock<D>::dma(Qp, ld, q0b, s, v, qk, lane);
      else if (t == 1) McBlock<D>::dma(Qp, ld, q0b, s, v, qm, lane);
      else if (t == 2) KcBlock<D>::dma(dOp, a, q0b, s, v, ok_, lane);
      else McBlock<D>::dma(dOp, a, q0b, s, v, om, lane);
    }
    // lse / delta of this wave's QPW queries: lanes [0, QPW/4) lse, [QPW/4, QPW/2) delta
    float *ldst = lslot(I) + wave * 256;
    constexpr int nl = QPW / 4;
    const float *src = lane < nl ? lp + q0b + wave * QPW + lane * 4
                                 : (lane < 2 * nl ? dp + q0b + wave * QPW + (lane - nl) * 4 : nullptr);
    dma16(src ? reinterpret_cast<const bf16_t *>(src) : zero_page(), reinterpret_cast<bf16_t *>(ldst));
  };
  auto compute = [&](auto I, int jj) {
    const int q0b = (jj + qstart) * BLK;
    if (kw >= s || (causal && kw > q0b + BLK - 1)) return;
    const bf16_t *qk = slot(0, I), *qm = slot(1, I), *ok_ = slot(2, I), *om = slot(3, I);
    const float *ls = lslot(I);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (causal && kw > q0b + sub * 32 + 31) continue;
      f32x16 sacc, dpacc;
      zero(sacc);
      zero(dpacc);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc = mfma32(KcBlock<D>::frag(qk, sub * 32 + l32, kk, hl), kf[kk], sacc);
        dpacc = mfma32(KcBlock<D>::frag(ok_, sub * 32 + l32, kk, hl), vf[kk], dpacc);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql0 = sub * 32 + g4 * 8 + hl * 4;
        const int w2 = ql0 / QPW, i0 = ql0 % QPW;
        const float4 L4 = *reinterpret_cast<const float4 *>(ls + w2 * 256 + i0);
        const float4 D4 = *reinterpret_cast<const float4 *>(ls + w2 * 256 + QPW + i0);
        const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = g4 * 4 + e, q = q0b + ql0 + e;
          float p = exp2f(sacc[r] * scale_log2 - Lv[e] * LOG2E);
          if (q >= s || (causal && kj > q)) p = 0.f;
          sacc[r] = p;
          dpacc[r] = p * (dpacc[r] - Dv[e]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8 pfr = acc_to_frag(sacc, hh), dsf = acc_to_frag(dpacc, hh);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          dv[t] = mfma32(McBlock<D>::frag_t(om, t * 32 + l32, sub * 32 + hh * 16, hl), pfr, dv[t]);
          dk[t] = mfma32(McBlock<D>::frag_t(qm, t * 32 + l32, sub * 32 + hh * 16, hl), dsf, dk[t]);
        }
      }
    }
  };
  pipeline<STAGES, DL, true>((s + BLK - 1) / BLK - qstart, issue, compute);

  if (kj < s) {
    bf16_t *pk = dqkv + (int64_t)(b * s + kj) * ld + a + h * D;
    bf16_t *pv = pk + a;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = t * 32 + jj * 8 + hl * 4;
        *reinterpret_cast<uint2 *>(pk + d0) =
            make_uint2(pack_bf16x2(dk[t][jj * 4 + 0] * scale, dk[t][jj * 4 + 1] * scale),
                       pack_bf16x2(dk[t][jj * 4 + 2] * scale, dk[t][jj * 4 + 3] * scale));
        *reinterpret_cast<uint2 *>(pv + d0) =
            make_uint2(pack_bf16x2(dv[t][jj * 4 + 0], dv[t][jj * 4 + 1]),
                       pack_bf16x2(dv[t][jj * 4 + 2], dv[t][jj * 4 + 3]));
      }
  }
}

template <int D, int STAGES>
__global__ void __launch_bounds__(64 * QP_NW)
    attn_bwd_dq_qp_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                          const float *__restrict__ lse, const float *__restrict__ delta,
                          bf16_t *__restrict__ dqkv, int s, int s_pad, int nh, int causal,
                          float scale_log2, float scale) {
  constexpr int NW = QP_NW, QT = 32 * NW, TE = BLK * D;
  constexpr int U = 3 * (D / 8);
  static_assert(U % NW == 0, "units per wave");
  constexpr int DL = U / NW;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[3 * STAGES * TE];
  auto slot = [&](int t, auto I) { return smem + (t * STAGES + decltype(I)::value) * TE; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int ntile = (s + QT - 1) / QT;
  const int q0 = (ntile - 1 - (int)blockIdx.x) * QT;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const int qw = q0 + wave * 32, qi = qw + l32;
  const bool qok = qi < s;

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qok ? load_frag(Qp + (int64_t)qi * ld + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    df[kk] = qok ? load_frag(dOp + (int64_t)qi * a + kk * 16 + hl * 8) : as_frag(make_uint4(0, 0, 0, 0));
    settle(qf[kk]);
    settle(df[kk]);
  }
  const float lq = qok ? lse[(int64_t)bh * s_pad + qi] * LOG2E : 0.f;
  const float dlt = qok ? delta[(int64_t)bh * s_pad + qi] : 0.f;
  settle(lq);
  settle(dlt);
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(dq[t]);

  auto issue = [&](auto I, int j) {
    bf16_t *kk_ = slot(0, I), *km = slot(1, I), *vk = slot(2, I);
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const int u = i * NW + wave, t = u / (D / 8), v = u % (D / 8);
      if (t == 0) KcBlock<D>::dma(Kp, ld, j * BLK, s, v, kk_, lane);
      else if (t == 1) McBlock<D>::dma(Kp, ld, j * BLK, s, v, km, lane);
      else KcBlock<D>::dma(Vp, ld, j * BLK, s, v, vk, lane);
    }
  };
  auto compute = [&](auto I, int j) {
    const int kb0 = j * BLK;
    if (qw >= s || (causal && kb0 > qw + 31)) return;
    const bf16_t *kk_ = slot(0, I), *km = slot(1, I), *vk = slot(2, I);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 sacc, dpacc;
      zero(sacc);
      zero(dpacc);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc = mfma32(KcBlock<D>::frag(kk_, sub * 32 + l32, kk, hl), qf[kk], sacc);
        dpacc = mfma32(KcBlock<D>::frag(vk, sub * 32 + l32, kk, hl), df[kk], dpacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + sub * 32 + acc_row(r, hl);
        float p = exp2f(sacc[r] * scale_log2 - lq);
        if (!qok || key >= s || (causal && key > qi)) p = 0.f;
        dpacc[r] = p * (dpacc[r] - dlt);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8 dsf = acc_to_frag(dpacc, hh);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          dq[t] = mfma32(McBlock<D>::frag_t(km, t * 32 + l32, sub * 32 + hh * 16, hl), dsf, dq[t]);
      }
    }
  };
  const int kend = causal ? min(s, q0 + QT) : s;
  pipeline<STAGES, DL, true>((kend + BLK - 1) / BLK, issue, compute);

  if (qok) {
    bf16_t *pq = dqkv + (int64_t)(b * s + qi) * ld + h * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = t * 32 + jj * 8 + hl * 4;
        *reinterpret_cast<uint2 *>(pq + d0) =
            make_uint2(pack_bf16x2(dq[t][jj * 4 + 0] * scale, dq[t][jj * 4 + 1] * scale),
                       pack_bf16x2(dq[t][jj * 4 + 2] * scale, dq[t][jj * 4 + 3] * scale));
      }
  }
}

// ---- launchers ---------------------------------------------------------------

int g_attn_variant = 0;  // 0 automatic, 1 split, 2 query-parallel

// query-parallel for long sequences (K/V reuse across 128 queries matters and
// there are enough 128-row tiles), split otherwise
bool use_qp(int s, int nbh) {
  if (g_attn_variant) return g_attn_variant == 2;
  return s >= 1024 && (int64_t)((s + 127) / 128) * nbh >= 128;
}

template <int D>
hipError_t fwd_d(int nb, int s, int nh, int causal, const void *qkv, void *o, float *lse, hipStream_t st) {
  const float scale_log2 = LOG2E / sqrtf((float)D);
  if (use_qp(s, nb * nh)) {
    dim3 grid((s + 32 * QP_NW - 1) / (32 * QP_NW), nb * nh);
    OASES_LAUNCH((attn_fwd_qp_kernel<D, 3>), grid, dim3(64 * QP_NW), st,
                       static_cast<const bf16_t *>(qkv), static_cast<bf16_t *>(o), lse, s, attn_lse_stride(s),
                       nh, causal, scale_log2);
  } else {
    dim3 grid((s + 31) / 32, nb * nh);
    OASES_LAUNCH((attn_fwd_kernel<D, 3>), grid, dim3(64 * Split<D>::NW), st,
                       static_cast<const bf16_t *>(qkv), static_cast<bf16_t *>(o), lse, s, attn_lse_stride(s),
                       nh, causal, scale_log2);
  }
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(int nb, int s, int nh, int causal, const void *qkv, const void *o, const void *dout,
                 const float *lse, float *delta, void *dqkv, hipStream_t st) {
  const int s_pad = attn_lse_stride(s);
  const int64_t rows = (int64_t)nb * s * nh;
  OASES_LAUNCH(attn_delta_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), st,
                     static_cast<const bf16_t *>(o), static_cast<const bf16_t *>(dout), delta, nb, s, s_pad, nh);
  const float scale = 1.f / sqrtf((float)D), scale_log2 = scale * LOG2E;
  const bf16_t *q = static_cast<const bf16_t *>(qkv), *d_o = static_cast<const bf16_t *>(dout);
  bf16_t *dq = static_cast<bf16_t *>(dqkv);
  if (use_qp(s, nb * nh)) {
    dim3 grid((s + 32 * QP_NW - 1) / (32 * QP_NW), nb * nh);
    constexpr int KV_STAGES = D == 128 ? 2 : 3;
    OASES_LAUNCH((attn_bwd_dkdv_qp_kernel<D, KV_STAGES>), grid, dim3(64 * QP_NW), st, q, d_o, lse,
                       delta, dq, s, s_pad, nh, causal, scale_log2, scale);
    OASES_LAUNCH((attn_bwd_dq_qp_kernel<D, 3>), grid, dim3(64 * QP_NW), st, q, d_o, lse, delta, dq, s,
                       s_pad, nh, causal, scale_log2, scale);
  } else {
    dim3 grid((s + 31) / 32, nb * nh);
    OASES_LAUNCH((attn_bwd_dkdv_kernel<D, 2>), grid, dim3(64 * Split<D>::NW), st, q, d_o, lse, delta,
                       dq, s, s_pad, nh, causal, scale_log2, scale);
    OASES_LAUNCH((attn_bwd_dq_kernel<D, 3>), grid, dim3(64 * Split<D>::NW), st, q, d_o, lse, delta, dq,
                       s, s_pad, nh, causal, scale_log2, scale);
  }
  return hipGetLastError();
}

}  // namespace

int attn_lse_stride(int s) { return (s + BLK - 1) / BLK * BLK; }

void attention_set_variant(int v) { g_attn_variant = v; }

template <int D>
hipError_t fwd_nw(int nw, int nb, int s, int nh, int causal, const void *qkv, void *o, float *lse, hipStream_t st) {
  if (nw == 4) return fwd_d<D, 4>(nb, s, nh, causal, qkv, o, lse, st);
  if (nw == 2) return fwd_d<D, 2>(nb, s, nh, causal, qkv, o, lse, st);
  return fwd_d<D, 1>(nb, s, nh, causal, qkv, o, lse, st);
}

template <int D>
hipError_t bwd_nw(int nw, int nb, int s, int nh, int causal, const void *qkv, const void *o, const void *dout,
                  const float *lse, float *delta, void *dqkv, hipStream_t st) {
  if (nw == 4) return bwd_d<D, 4>(nb, s, nh, causal, qkv, o, dout, lse, delta, dqkv, st);
  if (nw == 2) return bwd_d<D, 2>(nb, s, nh, causal, qkv, o, dout, lse, delta, dqkv, st);
  return bwd_d<D, 1>(nb, s, nh, causal, qkv, o, dout, lse, delta, dqkv, st);
}

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
