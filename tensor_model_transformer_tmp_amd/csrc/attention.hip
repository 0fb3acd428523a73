// Causal multi-head attention of the attention block's shard (bf16, MFMA).
//
// QKV is [nb*s, 3a] with columns [Q | K | V], each head-major (head h owns
// columns h*d .. h*d+d-1 of its part); O is [nb*s, a].  Per (sequence, head):
//   O = softmax(Q K^T / sqrt(d) + causal mask) V,   lse = log-sum-exp of a row.
// lse and delta are stored per (sequence, head) with a row stride of
// s_pad = s rounded up to 64.
//
// Work split.  The backward kernels run 4-wave workgroups, the forward 4 or
// 8 (two waves per SIMD where 8-wave workgroups alone give 256).  A wave owns
// 32 rows (queries for the forward and dQ, keys for dK/dV) and walks 32-row
// blocks of the other operand, staged in LDS by the gfx950 LDS DMA STAGES-1
// steps ahead.  The waves are OWN x SPLIT: OWN waves own different 32-row
// tiles and share the staged blocks; SPLIT waves own the same tile and take
// every SPLIT-th block of the walk, and their partial results are combined
// through LDS in wave order at the end (a fixed order: results are
// deterministic).  The host picks the largest OWN that still gives 256
// workgroups, so short sequences with few heads split the walk instead of
// leaving CUs idle.  Causal walks grow (forward, dQ) or shrink (dK/dV) with
// the tile index; when there are enough tiles, a backward workgroup takes
// two, one from each end, so all workgroups carry the same work.  Workgroup
// indices are permuted so that each XCD serves whole heads (wg_coords).
//
// The dK/dV kernel keeps its key tile's K and V in LDS (fragment-major, read
// with immediate offsets) rather than in registers, and addresses the staged
// Q and dO blocks through one base register each (the swizzle is an XOR):
// its dK and dV accumulators fill half the register file, and the rest must
// hold fragments in flight rather than hoisted addresses.
//
// Layout of a staged 32 x D block: row-major, 16-byte chunk c of row k at
// c ^ swz(k).  The swizzle keeps both reads conflict-free on the 64-bank LDS:
// the 16-byte row-fragment read (16 lanes, 16 consecutive rows, one chunk)
// and the transposing ds_read_b64_tr_b16 (4 consecutive rows x 4 chunks per
// 32 lanes), so each tensor is staged once and read both ways.
//
// Accumulator tiles are transposed so that a lane owns one row of the wave's
// tile (a query, or a key for dK/dV): softmax statistics are per-lane values
// plus one exchange with the lane 32 away (v_permlane32_swap), and a P / dS
// tile in accumulator layout is directly the B operand of the next MFMA once
// the A operand is read with the same (accumulator-row) order of its k index.
//
// The forward rescales its output accumulator lazily: the reference maximum
// of a row moves only when a new score exceeds it by more than 8 (log2
// units), so an unscaled probability is at most 2^8.  l and O share that
// reference, so the result is the same softmax; only the rounding differs.
//
// Backward (no atomics, five matmuls per block pair): a small kernel forms
// delta = rowsum(dO * O) per query; the dK/dV kernel then owns keys and walks
// query blocks (S = Q K^T, dP = dO V^T, P rebuilt from lse, dS = P (dP - delta),
// dV^T += dO^T P, dK^T += Q^T dS) and stores dS (bf16) in a scratch matrix
// [nb*n_h, s_pad, s_pad]; the dQ kernel owns queries and walks the key blocks
// of their causal range, staging K and dS blocks (dQ^T += K^T dS^T).  Every
// dS entry the dQ kernel reads was written by the dK/dV kernel (the causal
// lower triangle of 32 x 32 blocks, masked entries as zeros).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

constexpr int RB = 32;  // rows per staged block
constexpr int NW = 4;   // waves per workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr int LDS_BUDGET = 160 * 1024 - 2048;

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
// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// accumulator registers [8h, 8h+8) -> bf16 B-operand fragment
__device__ __forceinline__ bf16x8 acc_to_frag(const f32x16 &a, int h) {
  return as_frag(make_uint4(cvt_pk(a[8 * h + 0], a[8 * h + 1]), cvt_pk(a[8 * h + 2], a[8 * h + 3]),
                            cvt_pk(a[8 * h + 4], a[8 * h + 5]), cvt_pk(a[8 * h + 6], a[8 * h + 7])));
}
// row (within a 32-row MFMA tile) held in accumulator register r by lane half hl
__device__ __forceinline__ int acc_row(int r, int hl) { return (r >> 2) * 8 + hl * 4 + (r & 3); }
// value of x in lane (this lane ^ 32)
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// Workgroup coordinates of a (tiles x sequence-heads) grid, permuted so that
// the (sequence, head) index varies fastest over consecutive workgroups.
// Consecutive workgroups go to the 8 XCDs in turn, so when the number of
// (sequence, head) pairs is a multiple of 8 each XCD serves whole heads and
// its L2 holds their operands, instead of every XCD streaming every head.
__device__ __forceinline__ void wg_coords(int &x, int &bh) {
  const int lin = (int)(blockIdx.y * gridDim.x + blockIdx.x), nbh = (int)gridDim.y;
  bh = lin % nbh;
  x = lin / nbh;
}

// Make the compiler wait for (and keep) values loaded from global memory
// before the walk starts.  The LDS DMA is invisible to the compiler's wait
// counting, so a load still outstanding at the loop would otherwise be waited
// for inside the loop with a vmcnt that also drains the prefetch DMA.
__device__ __forceinline__ void settle(const bf16x8 &v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  asm volatile("" ::"v"(u));
}
__device__ __forceinline__ void settle(float v) { asm volatile("" ::"v"(v)); }

// ---- a staged block: 32 rows x D bf16 -----------------------------------------
template <int D>
struct Blk {
  static_assert(D == 64 || D == 128, "head size");
  static constexpr int BYTES = RB * D * 2;
  static constexpr int UNITS = BYTES / 1024;  // DMA instructions per block
  static constexpr int ELEMS = RB * D;
  __device__ __forceinline__ static int swz(int k) {
    if constexpr (D == 64) {
      const int a = (k >> 1) & 7;
      return a ^ ((a & 1) << 2);
    } else {
      return ((k & 3) << 2) | ((k >> 2) & 3);
    }
  }
  // source of lane `lane` in DMA unit u: row of the block and byte offset in the row
  __device__ __forceinline__ static void unit_src(int u, int lane, int &row, int &col_bytes) {
    const int byte = u * 1024 + lane * 16;
    row = byte / (2 * D);
    const int slot = (byte % (2 * D)) >> 4;
    col_bytes = (slot ^ swz(row)) << 4;
  }
  // row fragment: the 8 columns [kk*16 + hl*8, +8) of row `row`
  __device__ __forceinline__ static bf16x8 frag(const bf16_t *blk, int row, int kk, int hl) {
    return load_frag(blk + row * D + (((kk * 2 + hl) ^ swz(row)) << 3));
  }
  // Transposed fragment: column `col` at the 8 rows {k_lo + hl*4 + 0..3,
  // k_lo + 8 + hl*4 + 0..3} (the accumulator-row order of 16 rows from k_lo).
  // In each 16-lane group, source lane i addresses row base + i/4 at columns
  // col0 + 4 (i % 4); the transposing read hands lane i rows base..base+3 of
  // column col0 + i.
  __device__ __forceinline__ static bf16x8 frag_t(const bf16_t *blk, int col, int k_lo, int hl) {
    const int i = threadIdx.x & 15;
    const int n = (col - i) + 4 * (i & 3);
    v4i16 v[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = k_lo + r * 8 + hl * 4 + (i >> 2);
      const bf16_t *p = blk + k * D + (((n >> 3) ^ swz(k)) << 3) + (n & 7);
      v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(lds_void_t *)p);
    }
    const uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
    return as_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  // The same in natural row order: rows k_lo + hl*8 + 0..7 (the order of a
  // row-fragment read of 8 consecutive columns, e.g. of a dS row).
  __device__ __forceinline__ static bf16x8 frag_tn(const bf16_t *blk, int col, int k_lo, int hl) {
    const int i = threadIdx.x & 15;
    const int n = (col - i) + 4 * (i & 3);
    v4i16 v[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = k_lo + hl * 8 + r * 4 + (i >> 2);
      const bf16_t *p = blk + k * D + (((n >> 3) ^ swz(k)) << 3) + (n & 7);
      v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(lds_void_t *)p);
    }
    const uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
    return as_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }

  // The same reads from 32-bit LDS byte addresses.  The chunk swizzle is an
  // XOR, so the address of a lane's row fragment kk is its kk = 0 address
  // XOR (kk << 5), and that of a transposed fragment (column tile t, rows
  // 16 hh .. 16 hh + 15, half r of the read) is its (0, 0, 0) address XOR a
  // lane-independent mask, plus hh and r row offsets that become immediate
  // offsets of the read.  One base register per staged block serves every
  // fragment of it (a brute-force check over all lanes of these identities
  // is in the tests).
  __device__ __forceinline__ static uint32_t frag_base(uint32_t blk, int row, int hl) {
    return blk + row * D * 2 + ((hl ^ swz(row)) << 4);
  }
  __device__ __forceinline__ static bf16x8 frag_at(uint32_t base, int kk) {
    return lds_frag(base ^ (uint32_t)(kk << 5));
  }
  __device__ __forceinline__ static uint32_t frag_t_base(uint32_t blk, int hl) {
    const int lane = threadIdx.x & 63, i = lane & 15;
    const int n = (lane & 31) - i + 4 * (i & 3), k = hl * 4 + (i >> 2);
    return blk + k * D * 2 + ((((n >> 3) ^ swz(k)) << 3) + (n & 7)) * 2;
  }
  static constexpr uint32_t tmask(int t, int r) { return D == 128 ? ((t << 6) ^ (r << 5)) : (((t ^ r) & 1) << 6); }
  __device__ __forceinline__ static bf16x8 frag_t_at(uint32_t base, int t, int hh) {
    v4i16 v[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t a = (base ^ tmask(t, r)) + (uint32_t)((hh * 16 + r * 8) * D * 2);
      v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(uintptr_t)a);
    }
    const uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
    return as_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
};

// Walk steps 0..nst-1 through a ring of STAGES LDS slots.  issue(i, slot)
// starts the DMA of step i (exactly DL DMA instructions per wave);
// compute(i, slot) consumes it.  The barrier of step i also guarantees that
// every wave has finished step i-1, whose slot the DMA issued next reuses.
template <int STAGES, int DL, class Issue, class Compute>
__device__ __forceinline__ void walk(int nst, Issue &&issue, Compute &&compute) {
  static_assert(STAGES == 2 || STAGES == 3, "2 or 3 stages");
  if (nst <= 0) return;
  issue(0, 0);
  if constexpr (STAGES == 3)
    if (nst > 1) issue(1, 1);
  int slot = 0;
  for (int i = 0; i < nst; ++i) {
    if (STAGES == 3 && i + 1 < nst) wait_vmcnt<DL>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (i + STAGES - 1 < nst) {
      int ahead = slot + STAGES - 1;
      if (ahead >= STAGES) ahead -= STAGES;
      issue(i + STAGES - 1, ahead);
    }
    compute(i, slot);
    slot = slot + 1 == STAGES ? 0 : slot + 1;
  }
}

// a wave's [D x 32] accumulator tiles (rows d, columns = the wave's 32 rows) -> red
template <int D>
__device__ __forceinline__ void stash(float *red, const f32x16 (&acc)[D / 32], int l32, int hl) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(t * 32 + acc_row(r, hl)) * 32 + l32] = acc[t][r];
}

// Sum the SPLIT stashed partials of each owned tile in split order and store
// them as bf16 at row (row0 + own*32 + q), columns [d0, d0+8) of dst (row
// stride ld), times scale.  red holds [split][own][D][32] floats.
template <int D, int OWN, int SPLIT, int W = NW>
__device__ __forceinline__ void combine_store(const float *red, bf16_t *dst, int ld, int row0, int nrows,
                                              float scale) {
  for (int c = threadIdx.x; c < OWN * 32 * (D / 8); c += 64 * W) {
    const int q = c % 32, d0 = ((c / 32) % (D / 8)) * 8, own = c / (32 * (D / 8));
    const int row = row0 + own * 32 + q;
    if (row >= nrows) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int sp = 0; sp < SPLIT; ++sp) acc += red[((sp * OWN + own) * D + d0 + e) * 32 + q];
      o[e] = acc * scale;
    }
    *reinterpret_cast<uint4 *>(dst + (int64_t)row * ld + d0) =
        make_uint4(cvt_pk(o[0], o[1]), cvt_pk(o[2], o[3]), cvt_pk(o[4], o[5]), cvt_pk(o[6], o[7]));
  }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, int OWN, int W = NW>
struct KvCfg {  // staging of K and V blocks (forward); W waves per workgroup
  static constexpr int SPLIT = W / OWN;
  static constexpr int UNITS = SPLIT * 2 * Blk<D>::UNITS;  // K and V of SPLIT key blocks per step
  static_assert(UNITS % W == 0, "units per wave");
  static constexpr int DL = UNITS / W;
  static constexpr int STAGE_BYTES = SPLIT * 2 * Blk<D>::BYTES;
  static constexpr int STAGES = 3 * STAGE_BYTES <= LDS_BUDGET ? 3 : 2;
  static_assert(2 * STAGE_BYTES <= LDS_BUDGET, "two stages of K and V");
  static constexpr int RED_BYTES = W * D * 32 * 4 + W * 2 * 32 * 4;
  static constexpr int LDS = STAGES * STAGE_BYTES > RED_BYTES ? STAGES * STAGE_BYTES : RED_BYTES;
};

// Clamped DMA of one unit whose full-block source is base + voff bytes in a
// [rows x ld] matrix starting at row row0: rows past the last one read the
// last row (such rows are masked out of every result).
__device__ __forceinline__ void dma_clamped(const bf16_t *p, int ld, int row0, int rows, uint32_t voff,
                                            uint32_t lds) {
  const uint32_t e = voff >> 1, r = e / (uint32_t)ld, col = e - r * (uint32_t)ld;
  const int row = min(row0 + (int)r, rows - 1);
  dma16_v(p + (int64_t)row * ld + col, lds);
}

// K and V of SPLIT consecutive key blocks per step.  Unit uu = j*NW + wave of
// a step is block g = uu / (2 UNITS), K or V, unit uu % UNITS of that block.
// Lane offsets are relative to the step's first key row, so all units of a
// step share one scalar base and a unit costs a DMA and an M0 write.
template <int D, int OWN, int W = NW>
struct KvStager {
  using B = Blk<D>;
  using C = KvCfg<D, OWN, W>;
  uint32_t voff[C::DL];
  int lds[C::DL];  // byte offset of the unit in a stage (uniform)
  __device__ __forceinline__ void init(int wave, int lane, int ld, int a) {
#pragma unroll
    for (int j = 0; j < C::DL; ++j) {
      const int uu = j * W + wave, g = uu / (2 * B::UNITS), which = (uu / B::UNITS) & 1, u = uu % B::UNITS;
      int r, cb;
      B::unit_src(u, lane, r, cb);
      voff[j] = (uint32_t)(((g * RB + r) * ld + which * a) * 2 + cb);
      lds[j] = (g * 2 + which) * B::BYTES + u * 1024;
    }
  }
  // key rows [row0, row0 + SPLIT*RB) of K (V at column offset a) at Kp
  // stage: LDS byte address of the stage
  __device__ __forceinline__ void issue(const bf16_t *Kp, int ld, int s, int row0, uint32_t stage) const {
    if (row0 + C::SPLIT * RB <= s) {
      const bf16_t *base = Kp + (int64_t)row0 * ld;
#pragma unroll
      for (int j = 0; j < C::DL; ++j) dma16_s(base, voff[j], stage + lds[j]);
    } else {
#pragma unroll
      for (int j = 0; j < C::DL; ++j) dma_clamped(Kp, ld, row0, s, voff[j], stage + lds[j]);
    }
  }
};

template <int D, int OWN, int W>
__global__ void __launch_bounds__(64 * W)
    attn_fwd_kernel(const bf16_t *__restrict__ qkv, bf16_t *__restrict__ out, float *__restrict__ lse,
                    int s, int s_pad, int nh, int causal, float scale_log2, float scale, int pair) {
  using B = Blk<D>;
  using C = KvCfg<D, OWN, W>;
  constexpr int SPLIT = C::SPLIT, DL = C::DL;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  // pair == 2 (OWN == 2): the two owned 32-row tiles are the heavy tile
  // nt32-1-x and the light tile x of a causal walk, so every workgroup
  // carries the same work; waves 0..SPLIT-1 take the heavy tile and the
  // rest the light one, so that (waves being placed on the SIMDs in turn)
  // each SIMD runs one wave of each.  The light tile's keys are a prefix of
  // the heavy tile's, so both share every staged block.
  const bool hl_pair = OWN == 2 && pair == 2;
  const int own = hl_pair ? wave / SPLIT : wave % OWN, sp = hl_pair ? wave % SPLIT : wave / OWN;
  const int ntile = (s + 32 * OWN - 1) / (32 * OWN);
  const int nt32 = (s + 31) / 32;
  int wx, bh;
  wg_coords(wx, bh);
  const int b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a;

  KvStager<D, OWN, W> stg;
  stg.init(wave, lane, ld, a);

  // tiles of this workgroup, heaviest causal walk first: tile ntile-1-x, and
  // with pairing also tile x (equal work per workgroup)
  for (int rep = 0; rep < 1 + (pair == 1); ++rep) {
  const int tile = rep == 0 ? ntile - 1 - wx : wx;
  if (rep == 1 && tile >= ntile - 1 - wx) break;  // odd count: the middle tile is alone
  if (rep == 1) lds_barrier();  // the previous tile's combine has read the LDS
  // first row of owned tile ow; with hl_pair a light tile equal to the heavy
  // one (the middle of an odd count) is left to the heavy waves
  const int heavy = nt32 - 1 - wx, light = wx;
  auto row0_of = [&](int ow) { return hl_pair ? (ow == 0 ? heavy : light) * 32 : tile * 32 * OWN + ow * 32; };
  const bool idle = hl_pair && own == 1 && light >= heavy;
  const int q0 = hl_pair ? heavy * 32 : tile * 32 * OWN;  // the heavy (last) rows of the workgroup
  const int qw0 = row0_of(own), qi = qw0 + l32;

  bf16x8 qf[D / 16];
  {
    const int qrow = min(qi, s - 1);  // rows past the end compute on a real row; never stored
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = load_frag(Qp + (int64_t)qrow * ld + kk * 16 + hl * 8);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) settle(qf[kk]);
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(oacc[t]);
  float m_run = -INFINITY, l_run = 0.f;  // m_run: reference maximum of the raw scores
  const float slack = 8.f / scale_log2;

  const int kend = causal ? min(s, hl_pair ? q0 + 32 : q0 + 32 * OWN) : s;
  const int nkb = (kend + RB - 1) / RB;
  const int nst = (nkb + SPLIT - 1) / SPLIT;

  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int st, int slot) { stg.issue(Kp, ld, s, st * SPLIT * RB, smem_lds + slot * C::STAGE_BYTES); };
  auto compute = [&](int st, int slot) {
    const int kb = st * SPLIT + sp, k0 = kb * RB;
    if (idle || kb >= nkb || (causal && k0 > qw0 + 31)) return;
    const bf16_t *ks = reinterpret_cast<const bf16_t *>(smem + slot * C::STAGE_BYTES + sp * 2 * B::BYTES);
    const bf16_t *vs = ks + B::ELEMS;
    f32x16 sc;
    zero(sc);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) sc = mfma32(B::frag(ks, l32, kk, hl), qf[kk], sc);
    // sc[r] = S^T[key][q] (raw): key = k0 + acc_row(r, hl), q = qi
    if ((causal && k0 + 31 > qw0) || k0 + RB > s) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + acc_row(r, hl);
        if (key >= s || (causal && key > qi)) sc[r] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = fmaxf(mx, other_half(mx));
    const bool grow = mx > m_run + slack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? exp2_fast((m_run - mx) * scale_log2) : 1.f;  // m_run = -inf: 0
      if (grow) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
    }
    const float mc = m_run == -INFINITY ? 0.f : m_run * scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(sc[r], scale_log2, -mc));
      sc[r] = p;
      rs += p;
    }
    l_run += rs + other_half(rs);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 pf = acc_to_frag(sc, hh);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        oacc[t] = mfma32(B::frag_t(vs, t * 32 + l32, hh * 16, hl), pf, oacc[t]);
    }
  };
  walk<C::STAGES, DL>(nst, issue, compute);

  // combine the split waves' (m, l, O) per query in split order:
  //   O = sum_w 2^(m_w - m) O_w / sum_w 2^(m_w - m) l_w   (m in scaled units)
  lds_barrier();
  float *red = reinterpret_cast<float *>(smem);  // [split][own][D][32]
  float *ml = red + W * D * 32;                   // [split][own][2][32]
  stash<D>(red + (sp * OWN + own) * D * 32, oacc, l32, hl);
  if (hl == 0) {
    ml[((sp * OWN + own) * 2 + 0) * 32 + l32] = m_run;
    ml[((sp * OWN + own) * 2 + 1) * 32 + l32] = l_run;
  }
  lds_barrier();
  for (int c = threadIdx.x; c < OWN * 32 * (D / 8); c += 64 * W) {
    const int q = c % 32, d0 = ((c / 32) % (D / 8)) * 8, ow = c / (32 * (D / 8));
    const int qq = row0_of(ow) + q;
    if (qq >= s || (hl_pair && ow == 1 && light >= heavy)) continue;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) m = fmaxf(m, ml[((w * OWN + ow) * 2) * 32 + q]);
    float f[SPLIT], L = 0.f;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) {
      const float mw = ml[((w * OWN + ow) * 2) * 32 + q];
      f[w] = mw == -INFINITY ? 0.f : exp2_fast((mw - m) * scale_log2);
      L += f[w] * ml[((w * OWN + ow) * 2 + 1) * 32 + q];
    }
    const float inv = 1.f / L;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < SPLIT; ++w) acc += f[w] * red[((w * OWN + ow) * D + d0 + e) * 32 + q];
      o[e] = acc * inv;
    }
    *reinterpret_cast<uint4 *>(out + (int64_t)(b * s + qq) * a + h * D + d0) =
        make_uint4(cvt_pk(o[0], o[1]), cvt_pk(o[2], o[3]), cvt_pk(o[4], o[5]), cvt_pk(o[6], o[7]));
    if (d0 == 0) lse[(int64_t)bh * s_pad + qq] = m * scale + logf(L);
  }
  }
}

// ---------------------------------------------------------------------------
// backward: dK, dV.  A wave owns 32 keys and walks 32-query blocks of Q and dO
// (plus their lse and delta) from the first block its keys are visible to.
// ---------------------------------------------------------------------------
template <int D, int OWN>
struct DkdvCfg {
  static constexpr int SPLIT = NW / OWN;
  static constexpr int QU = SPLIT * Blk<D>::UNITS / NW;  // Q units per wave per step (dO: as many)
  static_assert(SPLIT * Blk<D>::UNITS % NW == 0, "units per wave");
  static constexpr int DL = 2 * QU + 1;                   // + one lse/delta (or padding) unit
  static constexpr int BLOCK_BYTES = 2 * Blk<D>::BYTES + 1024;
  static constexpr int STAGE_BYTES = SPLIT * BLOCK_BYTES + 1024;  // + a sink for padding units
  // K and V of the workgroup's OWN key tiles, staged once per tile above the ring
  static constexpr int KV_BYTES = OWN * 2 * Blk<D>::BYTES;
  static constexpr int KVU = KV_BYTES / 1024 / NW;  // their DMA units per wave
  static_assert(KV_BYTES % (1024 * NW) == 0, "K/V units per wave");
  static constexpr int STAGES = 3 * STAGE_BYTES + KV_BYTES <= LDS_BUDGET ? 3 : 2;
  static_assert(2 * STAGE_BYTES + KV_BYTES <= LDS_BUDGET, "two stages and the key tiles");
  static constexpr int KV_OFF = STAGES * STAGE_BYTES;
  static constexpr int RED_BYTES = NW * D * 32 * 4;
  static constexpr int LDS = KV_OFF + KV_BYTES > RED_BYTES ? KV_OFF + KV_BYTES : RED_BYTES;
  // a wave's consecutive DMA units are JROWS rows apart in the staged rows
  static constexpr int JROWS = NW * 1024 / (2 * D);
};

// Q and dO of SPLIT consecutive query blocks per step, and their lse and
// delta.  Q unit j of a wave is unit qu = j*NW + wave of the step (block
// qu / UNITS); dO units likewise; wave w < SPLIT also stages the lse (lanes
// 0-7) and delta (lanes 8-15) of block w, other waves a padding unit, so
// every wave issues DL units per step.  The step's rows are consecutive in
// memory, so a lane's source row in unit j is j*JROWS plus that of unit 0,
// at the same swizzled column: one lane offset per tensor, and a scalar
// base per unit.
template <int D, int OWN>
struct DkdvStager {
  using B = Blk<D>;
  using C = DkdvCfg<D, OWN>;
  uint32_t qoff, ooff;  // lane byte offset of unit 0 from the step's first row (Q, dO)
  int qlds[C::QU];      // byte offset of Q unit j in a stage (its dO unit: + B::BYTES)
  __device__ __forceinline__ void init(int wave, int lane, int ld, int a) {
    const int byte = wave * 1024 + lane * 16;  // unit 0 of this wave lies in block 0
    const int r = byte / (2 * D), slot = (byte % (2 * D)) >> 4;
    const int cb = (slot ^ B::swz(r)) << 4;
    qoff = (uint32_t)(r * ld * 2 + cb);
    ooff = (uint32_t)(r * a * 2 + cb);
#pragma unroll
    for (int j = 0; j < C::QU; ++j) {
      const int qu = j * NW + wave;
      qlds[j] = (qu / B::UNITS) * C::BLOCK_BYTES + (qu % B::UNITS) * 1024;
    }
  }
  // query rows [row0, row0 + SPLIT*RB); stage: LDS byte address of the stage
  __device__ __forceinline__ void issue(const bf16_t *Qp, const bf16_t *dOp, const float *lp, const float *dlp,
                                        int ld, int a, int s, int s_pad, int row0, uint32_t stage, int wave,
                                        int lane) const {
    if (row0 + C::SPLIT * RB <= s) {
      const bf16_t *bq = Qp + (int64_t)row0 * ld, *bo = dOp + (int64_t)row0 * a;
#pragma unroll
      for (int j = 0; j < C::QU; ++j) dma16_s(bq + (int64_t)j * C::JROWS * ld, qoff, stage + qlds[j]);
#pragma unroll
      for (int j = 0; j < C::QU; ++j) dma16_s(bo + (int64_t)j * C::JROWS * a, ooff, stage + qlds[j] + B::BYTES);
    } else {
#pragma unroll
      for (int j = 0; j < C::QU; ++j)
        dma_clamped(Qp, ld, row0, s, qoff + (uint32_t)(j * C::JROWS * ld * 2), stage + qlds[j]);
#pragma unroll
      for (int j = 0; j < C::QU; ++j)
        dma_clamped(dOp, a, row0, s, ooff + (uint32_t)(j * C::JROWS * a * 2), stage + qlds[j] + B::BYTES);
    }
    if (wave < C::SPLIT) {  // lse and delta rows are padded to s_pad
      const int i = lane & 15, r = min(row0 + wave * RB, s_pad - RB) + 4 * (i & 7);
      dma16_v((i < 8 ? lp : dlp) + r, stage + wave * C::BLOCK_BYTES + 2 * B::BYTES);
    } else {
      dma16_v(zero_page(), stage + C::SPLIT * C::BLOCK_BYTES);
    }
  }
};

template <int D, int OWN>
__global__ void __launch_bounds__(64 * NW)
    attn_dkdv_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout,
                     const float *__restrict__ lse, const float *__restrict__ delta,
                     bf16_t *__restrict__ dsm, bf16_t *__restrict__ dqkv, int s, int s_pad, int nh,
                     int causal, float scale_log2, float scale, int pair) {
  using B = Blk<D>;
  using C = DkdvCfg<D, OWN>;
  constexpr int SPLIT = C::SPLIT, DL = C::DL;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int own = wave % OWN, sp = wave / OWN;
  const int ntile = (s + 32 * OWN - 1) / (32 * OWN);
  // tiles of this workgroup, longest causal walk first: tile x, and with
  // pairing also tile ntile-1-x
  int wx, bh;
  wg_coords(wx, bh);
  for (int rep = 0; rep < 1 + pair; ++rep) {
  const int tile = rep == 0 ? wx : ntile - 1 - wx;
  if (rep == 1 && tile <= wx) break;  // odd count: the middle tile is alone
  if (rep == 1) lds_barrier();  // the previous tile's combine has read the LDS
  const int k0 = tile * 32 * OWN;
  const int kw0 = k0 + own * 32, kj = kw0 + l32;
  const int b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Qp = qkv + (int64_t)b * s * ld + h * D;
  const bf16_t *Kp = Qp + a, *Vp = Qp + 2 * a;
  const bf16_t *dOp = dout + (int64_t)b * s * a + h * D;
  const float *lp = lse + (int64_t)bh * s_pad, *dlp = delta + (int64_t)bh * s_pad;

  DkdvStager<D, OWN> stg;
  stg.init(wave, lane, ld, a);

  // K and V of the OWN key tiles above the ring, fragment-major: 1-KB unit
  // (own*2 + [K, V]) * D/16 + kk holds, at lane l, the 16 bytes of row l%32,
  // columns 16 kk + 8 (l/32) .. +8 (the lane's MFMA fragment kk), so a
  // fragment read is one base address plus an immediate offset.  Rows past
  // the sequence read the last row (their results are masked).  The walk's
  // first wait and barrier also cover this DMA: it is issued first.
  constexpr int KFR = D / 16;  // fragments (1-KB units) per K or V tile
  const uint32_t kv_lds = lds_addr(smem) + C::KV_OFF;
#pragma unroll
  for (int j = 0; j < C::KVU; ++j) {
    const int unit = j * NW + wave, blk = unit / KFR, kk = unit % KFR;
    const int row = min(k0 + (blk >> 1) * 32 + l32, s - 1);
    dma16_v(((blk & 1) ? Vp : Kp) + (int64_t)row * ld + kk * 16 + hl * 8, kv_lds + unit * 1024);
  }
  const uint32_t kva = kv_lds + own * 2 * KFR * 1024 + lane * 16;  // K fragment kk at + kk KB, V after K
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    zero(dv[t]);
    zero(dk[t]);
  }

  const int nqb = (s + RB - 1) / RB;
  const int qb0 = causal ? k0 / RB : 0;
  const int nst = (nqb - qb0 + SPLIT - 1) / SPLIT;

  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int st, int slot) {
    stg.issue(Qp, dOp, lp, dlp, ld, a, s, s_pad, (qb0 + st * SPLIT) * RB, smem_lds + slot * C::STAGE_BYTES,
              wave, lane);
  };
  auto compute = [&](int st, int slot) {
    const int qb = qb0 + st * SPLIT + sp, qs0 = qb * RB;
    if (qb >= nqb || (causal && qs0 + 31 < kw0)) return;
    const char *blk = smem + slot * C::STAGE_BYTES + sp * C::BLOCK_BYTES;
    const uint32_t blk_lds = smem_lds + slot * C::STAGE_BYTES + sp * C::BLOCK_BYTES;
    const uint32_t qa = B::frag_base(blk_lds, l32, hl);  // dO: + B::BYTES
    const uint32_t qta = B::frag_t_base(blk_lds, hl);     // dO: + B::BYTES
    const float *ls = reinterpret_cast<const float *>(blk + 2 * B::BYTES);  // lse [32], delta [32]
    f32x16 sc, dp;
    zero(sc);
    zero(dp);
    // fragments of substep kk+1 are read while the MFMAs of kk run
    bf16x8 fr[2][4];  // [buffer][Q, K, dO, V]
    auto read4 = [&](int kk, int buf) {
      fr[buf][0] = B::frag_at(qa, kk);
      fr[buf][1] = lds_frag(kva + kk * 1024);
      fr[buf][2] = B::frag_at(qa + B::BYTES, kk);
      fr[buf][3] = lds_frag(kva + (KFR + kk) * 1024);
    };
    read4(0, 0);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + 1 < D / 16) read4(kk + 1, (kk + 1) & 1);
      sc = mfma32(fr[kk & 1][0], fr[kk & 1][1], sc);  // S[q][key]
      dp = mfma32(fr[kk & 1][2], fr[kk & 1][3], dp);  // dP[q][key]
    }
    // masked: queries past the sequence, keys after the query (causal), and
    // keys past the sequence (lanes of a partial last key tile compute on a
    // clamped key; their dS entries are read by the dQ kernel, so they must
    // be zero)
    const bool edge = (causal && qs0 < kw0 + 31) || qs0 + RB > s || kw0 + RB > s;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 L4 = *reinterpret_cast<const float4 *>(ls + g * 8 + hl * 4);
      const float4 D4 = *reinterpret_cast<const float4 *>(ls + 32 + g * 8 + hl * 4);
      const float lv[4] = {L4.x, L4.y, L4.z, L4.w}, dl[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = g * 4 + e;
        float p = exp2_fast(fmaf(sc[r], scale_log2, -lv[e] * LOG2E));
        float ds = p * (dp[r] - dl[e]);
        if (edge) {
          const int q = qs0 + acc_row(r, hl);
          const bool ok = q < s && kj < s && (!causal || kj <= q);
          p = ok ? p : 0.f;
          ds = ok ? ds : 0.f;
        }
        sc[r] = p;
        dp[r] = ds;
      }
    }
    // dS[q][key] in bf16 for the dQ kernel.  A lane holds one key (column)
    // and 16 query rows; lanes 2i and 2i+1 (adjacent keys) trade one value
    // so that each stores two adjacent keys of one row in a 4-byte word: the
    // even lane row acc_row(r), the odd lane row acc_row(r) + 1.  Waves whose
    // keys start past the sequence store nothing (columns stay below s_pad).
    if (kw0 < s) {
      bf16_t *drow = dsm + ((int64_t)bh * s_pad + qs0) * s_pad + (kj & ~1);
      const bool odd = lane & 1;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float x = odd ? dp[r] : dp[r + 1];
        const float y = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
        const uint32_t w = odd ? cvt_pk(y, dp[r + 1]) : cvt_pk(dp[r], y);
        *reinterpret_cast<uint32_t *>(drow + (int64_t)(acc_row(r, hl) + (odd ? 1 : 0)) * s_pad) = w;
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 pf = acc_to_frag(sc, hh), dsf = acc_to_frag(dp, hh);
      // all transposed fragments of this half first, then its MFMAs
      bf16x8 fo[D / 32], fq[D / 32];
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        fo[t] = B::frag_t_at(qta + B::BYTES, t, hh);
        fq[t] = B::frag_t_at(qta, t, hh);
      }
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        dv[t] = mfma32(fo[t], pf, dv[t]);
        dk[t] = mfma32(fq[t], dsf, dk[t]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2 * (D / 32), 0);  // the transposed reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 32), 0);      // then the MFMAs
    }
  };
  walk<C::STAGES, DL>(nst, issue, compute);

  float *red = reinterpret_cast<float *>(smem);
  bf16_t *dK = dqkv + (int64_t)b * s * ld + a + h * D;
  lds_barrier();
  stash<D>(red + (sp * OWN + own) * D * 32, dv, l32, hl);
  lds_barrier();
  combine_store<D, OWN, SPLIT>(red, dK + a, ld, k0, s, 1.f);
  lds_barrier();
  stash<D>(red + (sp * OWN + own) * D * 32, dk, l32, hl);
  lds_barrier();
  combine_store<D, OWN, SPLIT>(red, dK, ld, k0, s, scale);
  }
}

// ---------------------------------------------------------------------------
// backward: delta = rowsum(dO * O) per query, float32.  A workgroup covers
// 256 / (D/8) query rows of one (sequence, head); D/8 lanes read a row's
// 16-byte chunks and add their products in a fixed butterfly order.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
    attn_delta_kernel(const bf16_t *__restrict__ o, const bf16_t *__restrict__ dout, float *__restrict__ delta,
                      int s, int s_pad, int nh) {
  constexpr int CPR = D / 8, ROWS = 256 / CPR;
  const int bh = blockIdx.y, b = bh / nh, h = bh % nh, a = nh * D;
  const int c = threadIdx.x % CPR, q = blockIdx.x * ROWS + threadIdx.x / CPR;
  float part = 0.f;
  if (q < s) {
    const int64_t off = (int64_t)(b * s + q) * a + h * D + c * 8;
    const uint4 x = *reinterpret_cast<const uint4 *>(o + off);
    const uint4 y = *reinterpret_cast<const uint4 *>(dout + off);
    part = lo_f32(x.x) * lo_f32(y.x) + hi_f32(x.x) * hi_f32(y.x) + lo_f32(x.y) * lo_f32(y.y) +
           hi_f32(x.y) * hi_f32(y.y) + lo_f32(x.z) * lo_f32(y.z) + hi_f32(x.z) * hi_f32(y.z) +
           lo_f32(x.w) * lo_f32(y.w) + hi_f32(x.w) * hi_f32(y.w);
  }
#pragma unroll
  for (int m = 1; m < CPR; m <<= 1) part += __shfl_xor(part, m);
  if (c == 0 && q < s) delta[(int64_t)bh * s_pad + q] = part;
}

// ---------------------------------------------------------------------------
// backward: dQ.  A wave owns 32 queries and walks the 32-key blocks of their
// causal range, staging K blocks and the matching 32 x 32 dS blocks (written
// by the dK/dV kernel): dQ^T += K^T dS^T, then dQ = scale * dS K.
// ---------------------------------------------------------------------------
template <int D, int OWN>
struct DqCfg {
  static constexpr int SPLIT = NW / OWN;
  static constexpr int KU = SPLIT * Blk<D>::UNITS;  // K units per step
  static constexpr int SU = OWN * SPLIT * 2;        // dS units per step (two per 32 x 32 block)
  static_assert((KU + SU) % NW == 0, "units per wave");
  static constexpr int DL = (KU + SU) / NW;
  static constexpr int K_BYTES = SPLIT * Blk<D>::BYTES;
  static constexpr int STAGE_BYTES = K_BYTES + OWN * SPLIT * 2048;
  static constexpr int STAGES = 3 * STAGE_BYTES <= LDS_BUDGET ? 3 : 2;
  static constexpr int RED_BYTES = NW * D * 32 * 4;
  static constexpr int LDS = STAGES * STAGE_BYTES > RED_BYTES ? STAGES * STAGE_BYTES : RED_BYTES;
};

// chunk swizzle of a staged 32 x 32 dS block (64-byte rows): 16-byte chunk c
// of row r at c ^ ds_swz(r), so a fragment read of 16 consecutive rows at one
// chunk touches distinct bank slots
__device__ __forceinline__ int ds_swz(int r) { return (r >> 2) & 3; }

template <int D, int OWN>
__global__ void __launch_bounds__(64 * NW)
    attn_dq_kernel(const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dsm, bf16_t *__restrict__ dqkv,
                   int s, int s_pad, int nh, int causal, float scale, int pair) {
  using B = Blk<D>;
  using C = DqCfg<D, OWN>;
  constexpr int SPLIT = C::SPLIT, DL = C::DL;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int own = wave % OWN, sp = wave / OWN;
  const int ntile = (s + 32 * OWN - 1) / (32 * OWN);
  int wx, bh;
  wg_coords(wx, bh);
  const int b = bh / nh, h = bh % nh;
  const int a = nh * D, ld = 3 * a;
  const bf16_t *Kp = qkv + (int64_t)b * s * ld + a + h * D;
  const bf16_t *dsb = dsm + (int64_t)bh * s_pad * s_pad;

  // DMA units of a step: unit uu = j*NW + wave; K units first (K block
  // uu / UNITS of the step), then dS units (block (own o, split p) =
  // (uu - KU) / 2, rows 16 (uu - KU) % 2 .. +15).  K offsets are relative
  // to the step's first key row; dS units keep their row in the tile, split
  // and source chunk.
  uint32_t koff[DL];
  int ldso[DL], drow[DL], dsp[DL], dcol[DL];
#pragma unroll
  for (int j = 0; j < DL; ++j) {
    const int uu = j * NW + wave;
    if (uu < C::KU) {
      const int g = uu / B::UNITS, u = uu % B::UNITS;
      int r, cb;
      B::unit_src(u, lane, r, cb);
      koff[j] = (uint32_t)((g * RB + r) * ld * 2 + cb);
      ldso[j] = g * B::BYTES + u * 1024;
      drow[j] = dsp[j] = dcol[j] = 0;
    } else {
      const int du = uu - C::KU, bi = du >> 1, u = du & 1;
      const int row = u * 16 + (lane >> 2);
      koff[j] = 0;
      drow[j] = (bi / SPLIT) * 32 + row;
      dsp[j] = bi % SPLIT;
      dcol[j] = ((lane & 3) ^ ds_swz(row)) << 3;
      ldso[j] = C::K_BYTES + bi * 2048 + u * 1024;
    }
  }

  // tiles as in the forward: ntile-1-x, and with pairing also x
  for (int rep = 0; rep < 1 + pair; ++rep) {
  const int tile = rep == 0 ? ntile - 1 - wx : wx;
  if (rep == 1 && tile >= ntile - 1 - wx) break;
  if (rep == 1) lds_barrier();  // the previous tile's combine has read the LDS
  const int q0 = tile * 32 * OWN;
  const int qw0 = q0 + own * 32;

  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(dq[t]);

  const int kend = causal ? min(s, q0 + 32 * OWN) : s;
  const int nkb = (kend + RB - 1) / RB;
  const int nst = (nkb + SPLIT - 1) / SPLIT;

  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int st, int slot) {
    const int row0 = st * SPLIT * RB;
    const uint32_t stage = smem_lds + slot * C::STAGE_BYTES;
    const bool full = row0 + SPLIT * RB <= s;
    const bf16_t *kbase = Kp + (int64_t)row0 * ld;
#pragma unroll
    for (int j = 0; j < DL; ++j) {
      if (j * NW + wave < C::KU) {  // uniform across the wave
        if (full) dma16_s(kbase, koff[j], stage + ldso[j]);
        else dma_clamped(Kp, ld, row0, s, koff[j], stage + ldso[j]);
      } else {
        // rows past the sequence and blocks past the walk read a valid
        // block; their results are never used
        const int q = min(q0 + drow[j], s - 1);
        const int kb = min(st * SPLIT + dsp[j], nkb - 1);
        dma16_v(dsb + (int64_t)q * s_pad + kb * RB + dcol[j], stage + ldso[j]);
      }
    }
  };
  auto compute = [&](int st, int slot) {
    const int kb = st * SPLIT + sp, k0 = kb * RB;
    if (kb >= nkb || (causal && k0 > qw0 + 31)) return;
    const char *stg = smem + slot * C::STAGE_BYTES;
    const bf16_t *ks = reinterpret_cast<const bf16_t *>(stg + sp * B::BYTES);
    const bf16_t *dss = reinterpret_cast<const bf16_t *>(stg + C::K_BYTES + (own * SPLIT + sp) * 2048);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // dS^T fragment: query l32, keys hh*16 + hl*8 .. +7 (one row chunk)
      const bf16x8 dsf = load_frag(dss + l32 * RB + (((hh * 2 + hl) ^ ds_swz(l32)) << 3));
#pragma unroll
      for (int t = 0; t < D / 32; ++t) dq[t] = mfma32(B::frag_tn(ks, t * 32 + l32, hh * 16, hl), dsf, dq[t]);
    }
  };
  walk<C::STAGES, DL>(nst, issue, compute);

  float *red = reinterpret_cast<float *>(smem);
  lds_barrier();
  stash<D>(red + (sp * OWN + own) * D * 32, dq, l32, hl);
  lds_barrier();
  combine_store<D, OWN, SPLIT>(red, dqkv + (int64_t)b * s * ld + h * D, ld, q0, s, scale);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int g_attn_variant = 0;  // 0 automatic; 1, 2, 3: OWN = 1, 4, 2; 4, 5: OWN = 1, 2 with tile pairs;
                         // 6, 7, 8: forward with 8 waves, OWN = 2, 4, 1; 9: forward with 8 waves,
                         // a heavy and a light tile per workgroup

struct AttnPlan {
  int own;
  int pair;   // 1: a workgroup takes two tiles, one of the longest and one of the shortest causal walks,
              // one after the other; 2 (forward, OWN 2): its two owned tiles are such a pair
  int waves;  // waves per workgroup (the forward also runs 8)
};

// OWN (waves of a workgroup that own distinct 32-row tiles): the largest
// that still gives 256 workgroups over all (sequence, head) pairs.  Causal
// walks grow with the tile index; for the backward kernels, when
// single-owner tiles paired heavy-with-light still give 256 workgroups,
// every workgroup takes a pair (equal work per workgroup instead of a
// longest walk twice the average); measured on MI355X, pairs help the
// backward by up to a fifth at s = 2048.  The causal forward with d = 128
// pairs within the workgroup instead: its two owned tiles are a heavy and a
// light one, sharing the staged blocks (one tile after the other measured
// slower there).
AttnPlan pick_plan(int s, int nbh, int causal, bool bwd, int d = 128) {
  switch (g_attn_variant) {
    case 1: return {1, 0, NW};
    case 2: return {4, 0, NW};
    case 3: return {2, 0, NW};
    case 4: return {1, 1, NW};
    case 5: return {2, 1, NW};
    case 6: if (!bwd) return {2, 0, 8}; break;
    case 7: if (!bwd) return {4, 0, 8}; break;
    case 8: if (!bwd) return {d == 64 ? 1 : 2, 0, 8}; break;  // 8 waves of one tile: d = 64 only (LDS)
    case 9: if (!bwd) return {2, 2, 8}; break;  // 8 waves, a heavy and a light causal tile
    default: break;
  }
  if (bwd && causal && (int64_t)((s + 31) / 32 / 2) * nbh >= 256) return {1, 1, NW};
  if (!bwd && causal && d == 128 && (int64_t)((s + 63) / 64) * nbh >= 128)
    return {2, 2, 8};  // a heavy and a light tile per 8-wave workgroup (measured: 11-17% faster
                       // at s = 1024-2048 than single-tile splits, also at 128 workgroups)
  if (!bwd) {
    // forward: 8-wave workgroups (two waves per SIMD; the walk split four
    // or eight ways) when they alone give 256 workgroups
    for (int own : {4, 2})
      if ((int64_t)((s + 32 * own - 1) / (32 * own)) * nbh >= 256) return {own, 0, 8};
    if (d == 64 && (int64_t)((s + 31) / 32) * nbh >= 256) return {1, 0, 8};
  }
  for (int own : {4, 2})
    if ((int64_t)((s + 32 * own - 1) / (32 * own)) * nbh >= 256) return {own, 0, NW};
  return {1, 0, NW};
}

// workgroups along a (sequence, head): one per tile, or one per pair of tiles
int tile_wgs(int s, int own, int pair) {
  const int ntile = (s + 32 * own - 1) / (32 * own);
  return pair ? (ntile + 1) / 2 : ntile;
}

template <int D, int OWN, int W = NW>
hipError_t fwd_launch(int nb, int s, int nh, int causal, int pair, const void *qkv, void *o, float *lse,
                      hipStream_t st) {
  const float scale = 1.f / sqrtf((float)D);
  const dim3 grid(tile_wgs(s, OWN, pair == 1), nb * nh);  // pair 2: one workgroup per OWN tiles
  OASES_LAUNCH((attn_fwd_kernel<D, OWN, W>), grid, dim3(64 * W), st, static_cast<const bf16_t *>(qkv),
               static_cast<bf16_t *>(o), lse, s, attn_lse_stride(s), nh, causal, scale * LOG2E, scale, pair);
  return hipSuccess;
}

// delta, then dK / dV (which writes dS), then dQ from dS
template <int D, int OWN>
hipError_t bwd_launch(int nb, int s, int nh, int causal, int pair, const void *qkv, const void *o,
                      const void *dout, const float *lse, float *delta, void *dsm, void *dqkv, hipStream_t st) {
  const float scale = 1.f / sqrtf((float)D);
  const int s_pad = attn_lse_stride(s);
  const bf16_t *q = static_cast<const bf16_t *>(qkv), *d_o = static_cast<const bf16_t *>(dout);
  bf16_t *dq = static_cast<bf16_t *>(dqkv), *ds = static_cast<bf16_t *>(dsm);
  constexpr int DROWS = 256 / (D / 8);
  OASES_LAUNCH((attn_delta_kernel<D>), dim3((s + DROWS - 1) / DROWS, nb * nh), dim3(256), st,
               static_cast<const bf16_t *>(o), d_o, delta, s, s_pad, nh);
  const dim3 grid(tile_wgs(s, OWN, pair), nb * nh);
  OASES_LAUNCH((attn_dkdv_kernel<D, OWN>), grid, dim3(64 * NW), st, q, d_o, lse,
               static_cast<const float *>(delta), ds, dq, s, s_pad, nh, causal, scale * LOG2E, scale, pair);
  OASES_LAUNCH((attn_dq_kernel<D, OWN>), grid, dim3(64 * NW), st, q, static_cast<const bf16_t *>(ds), dq, s,
               s_pad, nh, causal, scale, pair);
  return hipSuccess;
}

template <int D>
hipError_t fwd_d(int nb, int s, int nh, int causal, const void *qkv, void *o, float *lse, hipStream_t st) {
  const AttnPlan pl = pick_plan(s, nb * nh, causal, false, D);
  if (pl.waves == 8) {
    switch (pl.own) {
      case 4: return fwd_launch<D, 4, 8>(nb, s, nh, causal, 0, qkv, o, lse, st);
      case 2: return fwd_launch<D, 2, 8>(nb, s, nh, causal, pl.pair, qkv, o, lse, st);
      default:
        if constexpr (D == 64) return fwd_launch<D, 1, 8>(nb, s, nh, causal, 0, qkv, o, lse, st);
        return fwd_launch<D, 2, 8>(nb, s, nh, causal, 0, qkv, o, lse, st);
    }
  }
  switch (pl.own) {
    case 4: return fwd_launch<D, 4>(nb, s, nh, causal, pl.pair, qkv, o, lse, st);
    case 2: return fwd_launch<D, 2>(nb, s, nh, causal, pl.pair, qkv, o, lse, st);
    default: return fwd_launch<D, 1>(nb, s, nh, causal, pl.pair, qkv, o, lse, st);
  }
}

template <int D>
hipError_t bwd_d(int nb, int s, int nh, int causal, const void *qkv, const void *o, const void *dout,
                 const float *lse, float *delta, void *dsm, void *dqkv, hipStream_t st) {
  const AttnPlan pl = pick_plan(s, nb * nh, causal, true);
  switch (pl.own) {
    case 4: return bwd_launch<D, 4>(nb, s, nh, causal, pl.pair, qkv, o, dout, lse, delta, dsm, dqkv, st);
    case 2: return bwd_launch<D, 2>(nb, s, nh, causal, pl.pair, qkv, o, dout, lse, delta, dsm, dqkv, st);
    default: return bwd_launch<D, 1>(nb, s, nh, causal, pl.pair, qkv, o, dout, lse, delta, dsm, dqkv, st);
  }
}

}  // namespace

int attn_lse_stride(int s) { return (s + 63) / 64 * 64; }

void attention_set_variant(int v) { g_attn_variant = v; }

hipError_t attention_fwd(int nb, int s, int nh, int d, int causal, const void *qkv, void *o,
                         float *lse, hipStream_t st) {
  if (nb <= 0 || s <= 0 || nh <= 0) return hipSuccess;
  if (d == 64) return fwd_d<64>(nb, s, nh, causal, qkv, o, lse, st);
  if (d == 128) return fwd_d<128>(nb, s, nh, causal, qkv, o, lse, st);
  return hipErrorInvalidValue;
}

int64_t attn_ds_elems(int nb, int nh, int s) {
  const int64_t sp = attn_lse_stride(s);
  return (int64_t)nb * nh * sp * sp;
}

hipError_t attention_bwd(int nb, int s, int nh, int d, int causal, const void *qkv, const void *o,
                         const void *dout, const float *lse, float *delta, void *dsm, void *dqkv,
                         hipStream_t st) {
  if (nb <= 0 || s <= 0 || nh <= 0) return hipSuccess;
  if (d == 64) return bwd_d<64>(nb, s, nh, causal, qkv, o, dout, lse, delta, dsm, dqkv, st);
  if (d == 128) return bwd_d<128>(nb, s, nh, causal, qkv, o, dout, lse, delta, dsm, dqkv, st);
  return hipErrorInvalidValue;
}

}  // namespace oases
