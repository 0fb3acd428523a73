// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), float32
// accumulation, multi-stage LDS ring with 64-deep k tiles.
//
// Used for the column-parallel and row-parallel GEMMs of a TMP shard and for
// their data and weight gradients:
//   forward / recompute   C[T, N] = X[T, K] W[N, K]^T        (A KC, B KC)
//   data gradient         dX[T, K] = dC[T, N] W[N, K]         (A KC, B MC)
//   weight gradient       dW[N, K] = dC[T, N]^T X[T, K]       (A MC, B MC)
//
// Tiling: a workgroup of WGM x WGN waves (4 or 8) computes a BM x BN tile of
// C; the tile shape is chosen per problem (dispatch_tile).  Every operand
// tile goes HBM -> LDS by the gfx950 LDS DMA (global_load_lds_dwordx4),
// without passing through registers, into a ring of STAGES slots.  The k
// loop is software-pipelined: the barrier of each k tile, its first LDS
// reads and the DMA refilling the slot just consumed all sit under the
// previous tile's last MFMAs.
//   * k-contiguous operands (KC) are held as [rows][BK] bf16 with the 16-byte
//     chunks of row r XOR-swizzled (kc_key), so that the 16-byte fragment
//     reads of 16 consecutive rows hit distinct banks of the 64-bank LDS
//     (measured: no bank-conflict cycles).
//   * m/n-contiguous operands (MC) are stored as they are and read with the
//     gfx950 transposing LDS read (McTile).
// The MFMA computes the transposed tile C^T = B^T A^T, so a lane owns one row
// m of C and runs of four consecutive columns n; the epilogue writes them as
// 16-byte vectors.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace oases {
namespace {

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// EPI_F32 that also stores the column sums of A in GemmArgs::colsum
constexpr int EPI_F32_COLSUM = 16;

// A k tile is BK = 64 or 32 elements deep (a kernel template parameter): 64
// for the 2-3 stage pipelines, 32 to fit 4-5 stages of the largest tiles in
// the 160 KB of LDS.

// KC tile row swizzle: 16-byte chunk c of row r is stored at c ^ kc_key(r).
// 64-deep rows (128 B): (r ^ (r >> 3)) & 7 puts 16 consecutive rows' copies
// of one chunk in distinct 16-byte bank slots; 32-deep rows (64 B, four rows
// per 256-byte bank window): (r >> 2) & 3 does the same.
template <int BK>
__device__ __forceinline__ int kc_key(int row) {
  static_assert(BK == 64 || BK == 32, "k tile depth");
  return BK == 64 ? ((row ^ (row >> 3)) & 7) : ((row >> 2) & 3);
}

// ---- operand loaders ------------------------------------------------------
//
// Every operand tile goes HBM -> LDS by DMA, one 1-KB wave instruction at a
// time.  A loader precomputes each lane's byte offset from the tile's origin
// once per workgroup, so a k step issues all of a wave's units from one
// scalar base.  Rows (KC) or columns (MC) past the end of the matrix are
// clamped to the last one: they only feed rows / columns of C that are never
// stored.  A k tile reaching past K reads the zero page for k >= K, so
// partial k tiles are exact.

// KC tile: [ROWS][BK] (k contiguous), chunk c of row r stored at c ^ kc_key(r).
template <int ROWS, int NW, int BK>
struct KcTile {
  static constexpr int RPU = 512 / BK;  // rows per 1-KB DMA unit
  static constexpr int CPR = BK / 8;    // 16-byte chunks per row
  static_assert((ROWS / RPU) % NW == 0, "units per wave");
  static constexpr int PER_WAVE = ROWS / RPU / NW;  // DMA instructions per wave per stage
  uint32_t voff[PER_WAVE];  // lane byte offset from element (row0, k0) of the operand
  __device__ __forceinline__ void init(int ld, int row0, int rows_total, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = j * NW + wave;               // RPU-row block of the tile
      const int r = blk * RPU + lane / CPR;
      const int c = (lane % CPR) ^ kc_key<BK>(r);  // global chunk landing at LDS chunk lane % CPR
      const int row = min(row0 + r, rows_total - 1);
      voff[j] = (uint32_t)(((row - row0) * ld + c * 8) * 2);
    }
  }
  // tile: LDS byte address of the stage's tile
  __device__ __forceinline__ void issue(const bf16_t *p, int ld, int row0, int k0, int K, uint32_t tile,
                                        int wave, int lane) const {
    const bf16_t *base = p + (int64_t)row0 * ld + k0;
    if (k0 + BK <= K) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) dma16_s(base, voff[j], tile + (j * NW + wave) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int r = (j * NW + wave) * RPU + lane / CPR;
        const int c = (lane % CPR) ^ kc_key<BK>(r);
        dma16_v(k0 + c * 8 < K ? base + voff[j] / 2 : zero_page(), tile + (j * NW + wave) * 1024);
      }
    }
  }
  __device__ __forceinline__ static const bf16_t *tile_base(const bf16_t *p, int ld, int row0, int k0) {
    return p + (int64_t)row0 * ld + k0;
  }
  // unit j of a full k tile whose origin is `base`
  __device__ __forceinline__ void issue_unit(const bf16_t *base, int j, uint32_t tile, int wave) const {
    dma16_s(base, voff[j], tile + (j * NW + wave) * 1024);
  }
  // MFMA fragments: 8 consecutive k (half hl of substep ks) of a tile row.
  // The chunk swizzle is an XOR, so a lane addresses all its fragments from
  // one base, the LDS byte address of substep 0 of its first row: substep ks
  // is the base XOR (ks << 5), and for the row 32 i further down the key
  // changes by XOR 4 i when BK = 64 (bit 6 of the address for odd i; the key
  // of 32-deep rows is unchanged).  Row and slot offsets are multiples of 128
  // bytes, so they add as immediates.
  __device__ __forceinline__ static uint32_t frag_base(uint32_t tile, int row, int hl) {
    return tile + (uint32_t)(row * BK * 2 + ((hl ^ kc_key<BK>(row)) << 4));
  }
  __device__ __forceinline__ static bf16x8 frag_at(uint32_t base, int slot_off, int ks, int i) {
    const uint32_t x = (uint32_t)((ks << 5) ^ (BK == 64 ? (i & 1) << 6 : 0));
    return lds_frag((base ^ x) + slot_off + i * 32 * BK * 2);
  }
};

// MC tile: [BK k][ROWS] (row index contiguous), 16-byte chunk c of k-row k
// stored at c ^ mc_swz(k).  Fragments are read with the gfx950 transposing
// LDS read: in each 16-lane group, source lane s addresses k-row k0 + s/4 at
// columns n0 + 4 (s % 4); lane i of the group then receives k0..k0+3 of column
// n0 + i.  Two such reads give the 8 consecutive k of a KC fragment, so both
// tile kinds feed the same MFMA.  The swizzle spreads the 4 k-rows of a read
// over the four 64-byte quarters of the 256-byte bank space.
template <int ROWS, int NW, int BK>
struct McTile {
  static constexpr int ROW_BYTES = ROWS * 2;
  static_assert((BK * ROW_BYTES / 1024) % NW == 0, "units per wave");
  static constexpr int PER_WAVE = BK * ROW_BYTES / 1024 / NW;
  uint32_t voff[PER_WAVE];  // lane byte offset from element (k0, col0) of the operand
  __device__ __forceinline__ static int unit_k(int blk, int lane) { return (blk * 1024 + lane * 16) / ROW_BYTES; }
  __device__ __forceinline__ void init(int ld, int col0, int cols_total, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = j * NW + wave;               // 1-KB block of the tile
      const int byte = blk * 1024 + lane * 16;
      const int kr = byte / ROW_BYTES, cp = (byte % ROW_BYTES) >> 4;
      const int c = cp ^ mc_swz<ROWS>(kr);
      const int col = min(col0 + c * 8, cols_total - 8);  // cols_total is a multiple of 8
      voff[j] = (uint32_t)((kr * ld + (col - col0)) * 2);
    }
  }
  __device__ __forceinline__ void issue(const bf16_t *p, int ld, int col0, int k0, int K, uint32_t tile,
                                        int wave, int lane) const {
    const bf16_t *base = p + (int64_t)k0 * ld + col0;
    if (k0 + BK <= K) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) dma16_s(base, voff[j], tile + (j * NW + wave) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j)
        dma16_v(k0 + unit_k(j * NW + wave, lane) < K ? base + voff[j] / 2 : zero_page(),
                tile + (j * NW + wave) * 1024);
    }
  }
  __device__ __forceinline__ static const bf16_t *tile_base(const bf16_t *p, int ld, int col0, int k0) {
    return p + (int64_t)k0 * ld + col0;
  }
  __device__ __forceinline__ void issue_unit(const bf16_t *base, int j, uint32_t tile, int wave) const {
    dma16_s(base, voff[j], tile + (j * NW + wave) * 1024);
  }
  __device__ __forceinline__ static bf16x8 frag(const bf16_t *tile, int row, int ks, int hl) {
    // `row` is this lane's column of the operand (its m or n); the group's base is row - (lane & 15)
    const int lane = threadIdx.x & 63, s = lane & 15;
    const int n = (row - s) + 4 * (s & 3);
    v4i16 v[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = ks * 16 + hl * 8 + r * 4 + (s >> 2);
      const bf16_t *a = tile + k * ROWS + (((n >> 3) ^ mc_swz<ROWS>(k)) << 3) + (n & 7);
      v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(lds_void_t *)a);
    }
    const uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
};

template <int ROWS, int NW, Layout L, int BK>
using Tile = typename std::conditional<L == KC, KcTile<ROWS, NW, BK>, McTile<ROWS, NW, BK>>::type;

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- epilogue ---------------------------------------------------------------
//
// A lane owns, for each of its TM row groups i, one row m and TN*4 runs of four
// consecutive columns.  Every global load an epilogue needs for row group i
// (bias, the GeLU input, the old float32 C) is issued before any of its math
// or stores, so the group waits for memory once instead of once per run.
//
// bf16 results are stored 16 bytes per lane: lane l and lane l ^ 32 own the
// same row and the two 4-column halves of each 8-column group, so one
// exchange (v_permlane32_swap) per pair of runs gives each lane a whole
// group -- the even group of the pair to the lower half-wave, the odd one to
// the upper -- instead of an 8-byte store per run (measured on MI355X: the
// 8-byte stores drained a 2048 x 8192 bf16 C at about 3 TB/s).

// value of x in lane (this lane ^ 32)
__device__ __forceinline__ uint32_t other_half_u32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}

// store w (the lane's packed runs of row m) as 16-byte groups at base + m * ld
template <int TN>
__device__ __forceinline__ void store_bf16_row(bf16_t *base, int ld, int m, int N, const int (&ncol)[TN][4],
                                               const uint2 (&w)[TN][4]) {
  const int hl = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint2 a0 = w[j][2 * p], a1 = w[j][2 * p + 1];
      // the lower half-wave keeps columns 16p .. 16p+7 of the tile's 32 (its
      // run 2p, then the upper lane's run 2p); the upper one 16p+8 .. 16p+15
      const uint2 send = hl ? a0 : a1;
      const uint32_t rx = other_half_u32(send.x), ry = other_half_u32(send.y);
      const uint4 out = hl ? make_uint4(rx, ry, a1.x, a1.y) : make_uint4(a0.x, a0.y, rx, ry);
      const int n = ncol[j][2 * p] + 4 * hl;
      if (n < N) *reinterpret_cast<uint4 *>(base + (int64_t)m * ld + n) = out;
    }
}

template <int EPI, int TN>
__device__ __forceinline__ void epilogue_row(const GemmArgs &g, int m, const int (&ncol)[TN][4],
                                             float (&v)[TN][4][4]) {
  constexpr bool GELU = EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_TANH;
  constexpr bool GELU_BWD = EPI == EPI_GELU_BWD || EPI == EPI_GELU_BWD_TANH;
  constexpr bool TANH = EPI == EPI_BIAS_GELU_TANH || EPI == EPI_GELU_BWD_TANH;
  constexpr bool BIAS = EPI == EPI_BIAS || GELU;
  uint2 in[TN][4];  // bias or aux (bf16 x 4)
  float4 old[TN][4];
  uint2 out_w[TN][4] = {}, pre_w[TN][4] = {};  // packed bf16 results: C, and the GeLU input U
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n = ncol[j][jj];
      if (n >= g.N) continue;
      if constexpr (BIAS) in[j][jj] = *reinterpret_cast<const uint2 *>(static_cast<const bf16_t *>(g.bias) + n);
      if constexpr (GELU_BWD)
        in[j][jj] = *reinterpret_cast<const uint2 *>(static_cast<const bf16_t *>(g.aux) + (int64_t)m * g.ld_aux + n);
      if constexpr (EPI == EPI_F32)
        if (g.beta) old[j][jj] = *reinterpret_cast<const float4 *>(static_cast<float *>(g.C) + (int64_t)m * g.ldc + n);
    }
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n = ncol[j][jj];
      if (n >= g.N) continue;
      float *x = v[j][jj];
      if constexpr (EPI == EPI_F32) {
        float4 o = make_float4(x[0], x[1], x[2], x[3]);
        if (g.beta) { o.x += old[j][jj].x; o.y += old[j][jj].y; o.z += old[j][jj].z; o.w += old[j][jj].w; }
        *reinterpret_cast<float4 *>(static_cast<float *>(g.C) + (int64_t)m * g.ldc + n) = o;
        continue;
      }
      if constexpr (BIAS) {
        x[0] += lo_f32(in[j][jj].x); x[1] += hi_f32(in[j][jj].x);
        x[2] += lo_f32(in[j][jj].y); x[3] += hi_f32(in[j][jj].y);
      }
      if constexpr (GELU) {
        pre_w[j][jj] = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) x[ii] = TANH ? gelu_tanh_f(x[ii]) : gelu_f(x[ii]);
      }
      if constexpr (GELU_BWD) {
        const float u[4] = {lo_f32(in[j][jj].x), hi_f32(in[j][jj].x), lo_f32(in[j][jj].y), hi_f32(in[j][jj].y)};
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) x[ii] *= TANH ? gelu_tanh_grad_f(u[ii]) : gelu_grad_f(u[ii]);
      }
      out_w[j][jj] = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    }
  if constexpr (EPI != EPI_F32) {
    if constexpr (GELU)
      if (g.pre) store_bf16_row<TN>(static_cast<bf16_t *>(g.pre), g.ld_pre, m, g.N, ncol, pre_w);
    store_bf16_row<TN>(static_cast<bf16_t *>(g.C), g.ldc, m, g.N, ncol, out_w);
  }
}

// ---- AllReduce-point sum on extra workgroups of a GEMM launch --------------
//
// Workgroup w of g.sum.wgs streams vectors w*T + t, w*T + t + stride, ...
// (T threads, 8 bf16 per vector): all peers of UNROLL vectors are loaded four
// at a time before their adds, in the order own, peer 0, peer 1, ... with one
// rounding -- the arithmetic of the standalone sum kernel, so results are
// bit-identical to it.
__device__ __forceinline__ uint4 nt_load(const uint4 *p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void add8(float (&a)[8], const uint4 &b) {
  a[0] += lo_f32(b.x); a[1] += hi_f32(b.x); a[2] += lo_f32(b.y); a[3] += hi_f32(b.y);
  a[4] += lo_f32(b.z); a[5] += hi_f32(b.z); a[6] += lo_f32(b.w); a[7] += hi_f32(b.w);
}
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ void fused_sum(const FusedSum &f, int wg) {
  constexpr int UNROLL = 2;
  const int64_t stride = (int64_t)f.wgs * blockDim.x;
  const uint4 *own = static_cast<const uint4 *>(f.own);
  const uint4 *peers = static_cast<const uint4 *>(f.peers);
  const int64_t pstride = f.peer_stride / 8;
  for (int64_t v0 = (int64_t)wg * blockDim.x + threadIdx.x; v0 < f.nvec; v0 += stride * UNROLL) {
    float acc[UNROLL][8];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t v = v0 + u * stride;
      const uint4 a = v < f.nvec ? nt_load(own + v) : make_uint4(0, 0, 0, 0);
      acc[u][0] = lo_f32(a.x); acc[u][1] = hi_f32(a.x); acc[u][2] = lo_f32(a.y); acc[u][3] = hi_f32(a.y);
      acc[u][4] = lo_f32(a.z); acc[u][5] = hi_f32(a.z); acc[u][6] = lo_f32(a.w); acc[u][7] = hi_f32(a.w);
    }
    int k = 0;
    for (; k + 4 <= f.np; k += 4) {
      uint4 b[4][UNROLL];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int64_t v = v0 + u * stride;
          b[q][u] = v < f.nvec ? nt_load(peers + (k + q) * pstride + v) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) add8(acc[u], b[q][u]);
    }
    for (; k < f.np; ++k) {
      uint4 b[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t v = v0 + u * stride;
        b[u] = v < f.nvec ? nt_load(peers + k * pstride + v) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) add8(acc[u], b[u]);
    }
    uint4 *out = static_cast<uint4 *>(f.out);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t v = v0 + u * stride;
      if (v < f.nvec && f.tail.res)
        drop_res8(acc[u], reinterpret_cast<const uint4 *>(f.tail.res)[v], v, f.tail.seed, f.tail.layer,
                  f.tail.sb, f.tail.thr, f.tail.scale, f.tail.drop);
      if (v < f.nvec)
        out[v] = make_uint4(cvt_pk_bf16(acc[u][0], acc[u][1]), cvt_pk_bf16(acc[u][2], acc[u][3]),
                            cvt_pk_bf16(acc[u][4], acc[u][5]), cvt_pk_bf16(acc[u][6], acc[u][7]));
    }
  }
}

// ---- kernel -----------------------------------------------------------------

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// wait until at most n * DL of this wave's vector-memory operations are
// outstanding, for a runtime n in [0, NMAX]
template <int NMAX, int DL>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (NMAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= NMAX) wait_vmcnt<NMAX * DL>();
    else wait_vmcnt_upto<NMAX - 1, DL>(n);
  }
}

// KS k groups: the workgroup holds KS groups of WGM x WGN waves.  Group kg
// walks k tiles [kg * nk, (kg + 1) * nk) of the nk * KS tiles (the host only
// launches KS = 2 for an even tile count) through its own LDS ring, in step
// with the other group (one shared barrier per k step), so a CU keeps twice
// the operand bytes in flight for a tile of C.  Group 1 then hands its
// partial tile to group 0 through LDS, which adds it to its own in a fixed
// order (deterministic) and runs the epilogue.
template <int BM, int BN, int WGM, int WGN, int STAGES, int BK, int KS, Layout LA, Layout LB, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN * KS) gemm_bf16_kernel(GemmArgs g) {
  static_assert(STAGES >= 2 && STAGES <= 6, "2 to 6 stages");
  static_assert(KS == 1 || KS == 2, "one or two k groups");
  constexpr int NW = WGM * WGN;  // waves per k group
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile shape");
  using TA = Tile<BM, NW, LA, BK>;
  using TB = Tile<BN, NW, LB, BK>;
  constexpr int DL = TA::PER_WAVE + TB::PER_WAVE;  // DMA instructions per wave per stage
  static_assert((STAGES - 1) * DL < 64, "vmcnt range");
  static_assert(BK / 16 % 2 == 0, "even substep count");
  static_assert(STAGES * KS * (BM + BN) * BK * 2 <= 160 * 1024, "LDS");
  // LDS ring of STAGES slots per operand and k group, always indexed with
  // compile-time slot numbers (fragment reads get immediate offsets from the
  // group's base)
  constexpr int A_ELEMS = STAGES * KS * BM * BK;  // the A ring, then the B ring
  __shared__ __attribute__((aligned(1024))) bf16_t smem[STAGES * KS * (BM + BN) * BK];

  // the first g.sum.wgs workgroups run a fused AllReduce-point sum
  if ((int)blockIdx.x < g.sum.wgs) {
    fused_sum(g.sum, blockIdx.x);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = KS == 1 ? 0 : wave_wg / NW;  // k group
  const int wave = KS == 1 ? wave_wg : wave_wg % NW;  // wave within its group
  const int l32 = lane & 31, hl = lane >> 5;  // hl: which 32-lane half
  const int wm = wave % WGM, wn = wave / WGM;

  // tile order: workgroups i, i+8, ... run on one XCD; give them neighbouring
  // tiles, grouped 8 m-tiles at a time along n, so an XCD's L2 sees reuse
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x - g.sum.wgs;  // sum.wgs is a multiple of 8: XCD round robin unchanged
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  constexpr int GROUP = 8;
  const int group_span = GROUP * tiles_n;
  const int first_m = (bid / group_span) * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % group_span) % gsize;
  const int tn = (bid % group_span) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t *A = static_cast<const bf16_t *>(g.A);
  const bf16_t *B = static_cast<const bf16_t *>(g.B);
  const int nk = (g.K + BK - 1) / BK / KS;  // k tiles of this group
  const int kt0 = kg * nk;                  // its first k tile

  auto slotA = [&](auto I) -> bf16_t * { return smem + (decltype(I)::value * KS + kg) * BM * BK; };
  auto slotB = [&](auto I) -> bf16_t * { return smem + A_ELEMS + (decltype(I)::value * KS + kg) * BN * BK; };
  TA ta;
  TB tb;
  ta.init(g.lda, m0, g.M, wave, lane);
  tb.init(g.ldb, n0, g.N, wave, lane);
  auto issue = [&](auto I, int stage) {
    ta.issue(A, g.lda, m0, (kt0 + stage) * BK, g.K, lds_addr(slotA(I)), wave, lane);
    tb.issue(B, g.ldb, n0, (kt0 + stage) * BK, g.K, lds_addr(slotB(I)), wave, lane);
  };
  f32x16 acc[TN][TM];
  // column sums of A over k (bias gradient beside a weight gradient): every
  // wave adds up the A fragments it feeds the MFMAs, lane half hl holding
  // k = 8 hl .. 8 hl + 7 of each 16-k substep, and the waves of the first n
  // tile store them.  A compile-time variant: a runtime branch between the
  // MFMAs and the accumulator reads of the epilogue is not allowed here.
  constexpr bool COL = EPI == EPI_F32_COLSUM;
  float csum[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) csum[i] = 0.f;
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // the k loop, software-pipelined across k tiles.  The fragments of
  // substep ks+1 are read from LDS while the MFMAs of substep ks run.  In the
  // last substep of tile kt each wave waits for its DMA of tile kt+1, passes
  // the workgroup barrier (every wave has then also finished reading tile kt)
  // and reads tile kt+1's first fragments; tile kt's slot is refilled with
  // tile kt+STAGES while that substep's MFMAs run.  The LDS latency of a new
  // tile and the barrier thus sit under MFMAs, and every slot's tile is in
  // flight for STAGES-1 tiles.
  constexpr int NKS = BK / 16;  // k substeps per tile
  constexpr int MF = TM * TN;   // MFMAs per substep
  constexpr int RD = TM * (LA == KC ? 1 : 2) + TN * (LB == KC ? 1 : 2);  // LDS reads per substep
  const int nkf = min(nk, g.K / BK - kt0);  // this group's full k tiles
  static_for<0, STAGES>([&](auto I) {
    if (decltype(I)::value < nk) issue(I, decltype(I)::value);
  });
  bf16x8 xa[2][TM], wb[2][TN];
  uint32_t fa0 = 0, fb0 = 0;  // KC fragment bases (slot 0)
  if constexpr (LA == KC) fa0 = TA::frag_base(lds_addr(slotA(std::integral_constant<int, 0>{})), wm * WTM + l32, hl);
  if constexpr (LB == KC) fb0 = TB::frag_base(lds_addr(slotB(std::integral_constant<int, 0>{})), wn * WTN + l32, hl);
  auto read_frags = [&](auto I, int ks, int buf) __attribute__((always_inline)) {
    constexpr int SI = decltype(I)::value;
#pragma unroll
    for (int i2 = 0; i2 < TM; ++i2) {
      if constexpr (LA == KC) xa[buf][i2] = TA::frag_at(fa0, SI * KS * BM * BK * 2, ks, i2);
      else xa[buf][i2] = TA::frag(slotA(I), wm * WTM + i2 * 32 + l32, ks, hl);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (LB == KC) wb[buf][j] = TB::frag_at(fb0, SI * KS * BN * BK * 2, ks, j);
      else wb[buf][j] = TB::frag(slotB(I), wn * WTN + j * 32 + l32, ks, hl);
    }
  };
  auto mfma_one = [&](int buf, int j, int i2) __attribute__((always_inline)) {
    acc[j][i2] = mfma32(wb[buf][j], xa[buf][i2], acc[j][i2]);
  };
  auto colsum = [&](int buf) __attribute__((always_inline)) {
    if constexpr (COL) {
      const bf16x2v one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int i2 = 0; i2 < TM; ++i2) {
        const uint4 u = __builtin_bit_cast(uint4, xa[buf][i2]);
        float c = csum[i2];
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u.x), one, c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u.y), one, c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u.z), one, c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u.w), one, c, false);
        csum[i2] = c;
      }
    }
  };
  wait_vmcnt_upto<STAGES - 1, DL>(min(STAGES - 1, nk - 1));  // tile 0 landed
  lds_barrier();
  read_frags(std::integral_constant<int, 0>{}, 0, 0);
  // one k tile in slot I.  FULL: tile kt+STAGES exists and is a full k tile,
  // so its DMA goes out a unit at a time between the last substep's MFMAs
  auto step = [&](auto I, int kt, auto FULL) __attribute__((always_inline)) {
    using NEXT = std::integral_constant<int, (decltype(I)::value + 1) % STAGES>;
    static_for<0, NKS>([&](auto KSUB) {
      constexpr int ks = decltype(KSUB)::value, cur = ks & 1;
      if constexpr (ks + 1 < NKS) {
        read_frags(I, ks + 1, cur ^ 1);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i2 = 0; i2 < TM; ++i2) mfma_one(cur, j, i2);
        colsum(cur);
        // each MFMA followed by its share of the next substep's reads
        constexpr int PER = (RD + MF - 1) / MF;
#pragma unroll
        for (int t = 0; t < MF; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (t * PER + q < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else if constexpr (decltype(FULL)::value) {
        wait_vmcnt<(STAGES - 2) * DL>();  // tile kt+1 landed
        lds_barrier();
        read_frags(NEXT{}, 0, 0);
        const int k0 = (kt0 + kt + STAGES) * BK;
        const bf16_t *ba = TA::tile_base(A, g.lda, m0, k0);
        const bf16_t *bb = TB::tile_base(B, g.ldb, n0, k0);
        const uint32_t la = lds_addr(slotA(I)), lb = lds_addr(slotB(I));
        static_for<0, MF>([&](auto T) {
          constexpr int t = decltype(T)::value;
          mfma_one(cur, t / TM, t % TM);
          // the DL units of the tile spread evenly over the MF MFMAs
          static_for<t * DL / MF, (t + 1) * DL / MF>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if constexpr (u < TA::PER_WAVE) ta.issue_unit(ba, u, la, wave);
            else tb.issue_unit(bb, u - TA::PER_WAVE, lb, wave);
          });
        });
        colsum(cur);
      } else {
        if (kt + 1 < nk) {
          wait_vmcnt_upto<STAGES - 2, DL>(min(STAGES - 2, nk - 2 - kt));  // tile kt+1 landed
          lds_barrier();
          if (kt + STAGES < nk) issue(I, kt + STAGES);
          read_frags(NEXT{}, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i2 = 0; i2 < TM; ++i2) mfma_one(cur, j, i2);
        colsum(cur);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // groups of STAGES k tiles (slots 0..STAGES-1 in order): first those whose
  // refills are full tiles, then the rest, then the tail
  int kt = 0;
  for (; kt + 2 * STAGES <= nkf; kt += STAGES)
    static_for<0, STAGES>([&](auto I) { step(I, kt + decltype(I)::value, std::true_type{}); });
  for (; kt + STAGES <= nk; kt += STAGES)
    static_for<0, STAGES>([&](auto I) { step(I, kt + decltype(I)::value, std::false_type{}); });
  static_for<0, STAGES - 1>([&](auto I) {
    if (kt + decltype(I)::value < nk) step(I, kt + decltype(I)::value, std::false_type{});
  });

  if constexpr (KS == 2) {
    // group 1's partial tile (and column sums) to group 0 through LDS; the
    // ring is free once every wave has passed this barrier
    constexpr int NT = NW * 64;  // threads of a group
    static_assert((TN * TM * 16 + TM) * NT * 4 <= (int)sizeof(smem), "reduction buffer");
    float *red = reinterpret_cast<float *>(smem);
    const int t = wave * 64 + lane;
    lds_barrier();
    if (kg == 1) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((j * TM + i) * 16 + r) * NT + t] = acc[j][i][r];
      if constexpr (COL) {
#pragma unroll
        for (int i = 0; i < TM; ++i) red[(TN * TM * 16 + i) * NT + t] = csum[i];
      }
    }
    lds_barrier();
    if (kg == 1) return;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] += red[((j * TM + i) * 16 + r) * NT + t];
    if constexpr (COL) {
#pragma unroll
      for (int i = 0; i < TM; ++i) csum[i] += red[(TN * TM * 16 + i) * NT + t];
    }
  }

  // epilogue: acc[j][i][jj*4 + ii] is C[m][n] with
  //   m = m0 + wm*WTM + i*32 + l32,  n = n0 + wn*WTN + j*32 + jj*8 + hl*4 + ii
  int ncol[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ncol[j][jj] = n0 + wn * WTN + j * 32 + jj * 8 + hl * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WTM + i * 32 + l32;
    if (m >= g.M) continue;
    float v[TN][4][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[j][jj][ii] = acc[j][i][jj * 4 + ii];
    epilogue_row<COL ? (int)EPI_F32 : EPI, TN>(g, m, ncol, v);
  }
  if constexpr (COL) {
    if (tn == 0 && wn == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float total = csum[i] + __shfl_xor(csum[i], 32);  // k halves 0..7 + 8..15
        const int m = m0 + wm * WTM + i * 32 + l32;
        if (hl == 0 && m < g.M) g.colsum[m] = (g.beta ? g.colsum[m] : 0.f) + total;
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int STAGES, Layout LA, Layout LB, int EPI, int BK = 64, int KS = 1>
hipError_t launch(const GemmArgs &g, hipStream_t s) {
  if constexpr (KS > 1) {  // k groups need an equal number of k tiles each
    if (((g.K + BK - 1) / BK) % KS != 0) return launch<BM, BN, WGM, WGN, STAGES, LA, LB, EPI, BK, 1>(g, s);
  }
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  OASES_LAUNCH((gemm_bf16_kernel<BM, BN, WGM, WGN, STAGES, BK, KS, LA, LB, EPI>), dim3(tiles + g.sum.wgs),
                     dim3(64 * WGM * WGN * KS), s, g);
  return hipGetLastError();
}

int g_variant = 0;  // 0 = automatic tile choice; >0 forces one (tuning sweeps)

template <Layout LA, Layout LB, int EPI>
hipError_t dispatch_tile(const GemmArgs &g, hipStream_t s) {
  int v = g_variant;
  if (v == 0) {
    // measured on MI355X over the workload shapes: 256x256 (8 waves) when it
    // alone gives a tile per CU, 128x256 (8 waves) near that; 128x128 tiles
    // (3 stages for long k loops, 2 stages for short) while they still give
    // a tile per CU, and below that 64x128 tiles (128x64 for a weight
    // gradient wider than it is tall), 4 stages deep for k >= 4096 (8-wave
    // 128x128 tiles when those nearly cover the CUs); short-k problems that
    // 64x64 tiles cover in at most two rounds run on 4-stage 64x64 tiles
    // (with the two sub-batches' GEMMs running side by side, the deeper ring
    // measured 5% faster over the 1024-hidden step).  Large weight gradients
    // wider than they are tall run best on 2-stage 128x128.  Measured with
    // two k groups (hipGraph replays): the 1024-hidden weight gradients
    // (k = 2048 tokens) 12.2-13.2 -> 9.7-10.7 us, the 4096-hidden
    // out-projection data gradient (2048x512, k = 4096) 24.2 -> 16.7 us.
    const int64_t t256 = (int64_t)((g.M + 255) / 256) * ((g.N + 255) / 256);
    const int64_t t128x256 = (int64_t)((g.M + 127) / 128) * ((g.N + 255) / 256);
    const int64_t t128 = (int64_t)((g.M + 127) / 128) * ((g.N + 127) / 128);
    const int64_t t64 = (int64_t)((g.M + 63) / 64) * ((g.N + 63) / 64);
    const int64_t t64x128 = (int64_t)((g.M + 63) / 64) * ((g.N + 127) / 128);
    const bool wide_dw = LA == MC && g.M < g.N;
    // long k loops over too few tiles for two workgroups per CU: two k groups
    // per tile (an even k-tile count, at least 16) -- 64x64 tiles while they
    // give at most one tile per CU, else 64x128 while those do
    const int nk64 = (g.K + 63) / 64;
    const bool ks2 = nk64 % 2 == 0 && nk64 >= 16;
    if (wide_dw && t128 >= 1024) v = 5;
    else if (t256 >= 256) v = 4;
    else if (t128x256 >= 192) v = 3;
    else if (t128 < 256 && ks2 && t64 <= 256) v = 20;
    else if (t128 < 256 && ks2 && t64x128 <= 256) v = 21;
    else if (t128 < 256 && g.K >= 4096) v = t128 >= 192 ? 13 : (wide_dw ? 12 : 9);
    else if (t128 < 256) v = t64 <= 512 ? 19 : (wide_dw ? 8 : 7);
    else if (g.K >= 2048) v = 2;
    else v = 5;
  }
  switch (v) {
    case 1: return launch<256, 128, 4, 2, 3, LA, LB, EPI>(g, s);
    case 2: return launch<128, 128, 2, 2, 3, LA, LB, EPI>(g, s);
    case 3: return launch<128, 256, 2, 4, 3, LA, LB, EPI>(g, s);
    case 4: return launch<256, 256, 4, 2, 2, LA, LB, EPI>(g, s);
    case 5: return launch<128, 128, 2, 2, 2, LA, LB, EPI>(g, s);
    case 6: return launch<256, 256, 2, 4, 2, LA, LB, EPI>(g, s);
    case 7: return launch<64, 128, 2, 2, 2, LA, LB, EPI>(g, s);
    case 8: return launch<128, 64, 2, 2, 2, LA, LB, EPI>(g, s);
    case 9: return launch<64, 128, 2, 2, 4, LA, LB, EPI>(g, s);
    case 10: return launch<64, 128, 2, 2, 6, LA, LB, EPI>(g, s);
    case 11: return launch<128, 128, 2, 2, 4, LA, LB, EPI>(g, s);
    case 12: return launch<128, 64, 2, 2, 4, LA, LB, EPI>(g, s);
    case 13: return launch<128, 128, 4, 2, 4, LA, LB, EPI>(g, s);
    case 14: return launch<256, 256, 4, 2, 4, LA, LB, EPI, 32>(g, s);
    case 15: return launch<256, 256, 4, 2, 5, LA, LB, EPI, 32>(g, s);
    case 16: return launch<128, 256, 2, 4, 5, LA, LB, EPI, 32>(g, s);
    case 17: return launch<256, 128, 4, 2, 5, LA, LB, EPI, 32>(g, s);
    case 18: return launch<64, 64, 2, 2, 2, LA, LB, EPI>(g, s);
    case 19: return launch<64, 64, 2, 2, 4, LA, LB, EPI>(g, s);
    // two k groups (an odd k-tile count runs the same tile with one group)
    case 20: return launch<64, 64, 2, 2, 4, LA, LB, EPI, 64, 2>(g, s);
    case 21: return launch<64, 128, 2, 2, 3, LA, LB, EPI, 64, 2>(g, s);
    case 22: return launch<128, 128, 2, 2, 2, LA, LB, EPI, 64, 2>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

void gemm_bf16_set_variant(int v) { g_variant = v; }

hipError_t gemm_bf16(Layout la, Layout lb, Epi epi, const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (la == KC && lb == KC) {
    switch (epi) {
      case EPI_STORE: return dispatch_tile<KC, KC, EPI_STORE>(g, s);
      case EPI_BIAS: return dispatch_tile<KC, KC, EPI_BIAS>(g, s);
      case EPI_BIAS_GELU: return dispatch_tile<KC, KC, EPI_BIAS_GELU>(g, s);
      case EPI_BIAS_GELU_TANH: return dispatch_tile<KC, KC, EPI_BIAS_GELU_TANH>(g, s);
      default: break;
    }
  } else if (la == KC && lb == MC) {
    switch (epi) {
      case EPI_STORE: return dispatch_tile<KC, MC, EPI_STORE>(g, s);
      case EPI_GELU_BWD: return dispatch_tile<KC, MC, EPI_GELU_BWD>(g, s);
      case EPI_GELU_BWD_TANH: return dispatch_tile<KC, MC, EPI_GELU_BWD_TANH>(g, s);
      default: break;
    }
  } else if (la == MC && lb == MC) {
    if (epi == EPI_F32)
      return g.colsum ? dispatch_tile<MC, MC, EPI_F32_COLSUM>(g, s) : dispatch_tile<MC, MC, EPI_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace oases
