// Host-side launchers of the gfx950 kernels.  Every launcher enqueues on
// `stream` and returns the hipError_t of the launch.  Shapes are checked by
// the caller (executor / C-ABI entry points) before any launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace oases {

// Kernel timing.  While a pair of events is armed (the executor arms one pair
// around each launch of the kernel class being timed), launches carry the
// events in their own dispatch packets: the start event takes the start time
// of the first kernel launched, the stop event the end time of every kernel
// launched (the last one wins).  The pair therefore spans exactly the class's
// kernels, with no marker packets of its own in the stream.
struct LaunchTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTimer &launch_timer();  // per host thread

template <class K, class... Args>
inline hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  LaunchTimer &t = launch_timer();
  if (t.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t.start, t.stop, 0, args...);
    t.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
  return hipGetLastError();
}

// launch through launch_kernel and return its error from the enclosing function
#define OASES_LAUNCH(kernel, grid, block, stream, ...)                                    \
  do {                                                                                   \
    if (hipError_t oases_launch_err_ = ::oases::launch_kernel(kernel, grid, block, stream, \
                                                              __VA_ARGS__))              \
      return oases_launch_err_;                                                          \
  } while (0)

// GEMM epilogues
enum Epi : int {
  EPI_STORE = 0,      // C = acc                              (storage type)
  EPI_BIAS = 1,       // C = acc + bias[n]
  EPI_BIAS_GELU = 2,  // pre = acc + bias[n] (optional), C = gelu(acc + bias[n])
  EPI_GELU_BWD = 3,   // C = acc * gelu'(aux[m][n])
  EPI_F32 = 4,        // C(float32) = acc (+ C if beta)
  EPI_BIAS_GELU_TANH = 6,  // EPI_BIAS_GELU with the tanh form of GeLU (bf16)
  EPI_GELU_BWD_TANH = 7    // EPI_GELU_BWD with the tanh form of GeLU (bf16)
};

// Operand layouts: for A(m,k): KC = stored [M][lda] (k contiguous),
// MC = stored [K][lda] (m contiguous).  For B(k,n): KC = stored [N][ldb]
// (k contiguous), MC = stored [K][ldb] (n contiguous).
enum Layout : int { KC = 0, MC = 1 };

// An AllReduce-point sum (out = own + peers[0..np), float32 adds in that
// order, one rounding) that a GEMM launch runs on extra workgroups beside its
// tiles (sum_wgs of them; none when 0).  Same arithmetic as allreduce_point.
// Replicated tail of a full transformer block applied to an AllReduce
// point's sum S (bf16): out = res + dropout(S), elementwise.  Element e of the
// [T_sb, h] sub-batch buffer is kept iff output word e % 4 of
// Philox4x64-10 at counter (e / 4, sb, 0, 0) under key (seed, layer) is
// below thr; kept elements are scaled by `scale` = 1 / (1 - p).  res null:
// no tail (out = S).  drop 0: no dropout (out = res + S).
struct DropRes {
  const void *res;
  uint64_t seed, layer, sb, thr;
  float scale;
  int drop;
};

struct FusedSum {
  const void *own;
  const void *peers;
  int64_t peer_stride;  // elements between peers
  void *out;
  int64_t nvec;         // 8-element vectors (n / 8)
  int np;
  int wgs;
  DropRes tail;  // res null: none
};

struct GemmArgs {
  int M, N, K;
  const void *A;
  int lda;
  const void *B;
  int ldb;
  void *C;
  int ldc;
  const void *bias;
  void *pre;
  int ld_pre;
  const void *aux;
  int ld_aux;
  int beta;
  FusedSum sum;  // bf16 GEMMs only
  // bf16 GEMMs with A stored [K][lda] (m contiguous) only: colsum[m] =
  // (beta ? colsum[m] : 0) + sum over k of A(m, k), float32 -- the bias
  // gradient of a weight-gradient GEMM (none when null)
  float *colsum;
};

// C[M,N] = sum_k A(m,k) B(k,n) with the given layouts and epilogue.
// bf16 operands on MFMA; float32 operands on a SIMT kernel.
hipError_t gemm_bf16(Layout la, Layout lb, Epi epi, const GemmArgs &g, hipStream_t s);
hipError_t gemm_f32(Layout la, Layout lb, Epi epi, const GemmArgs &g, hipStream_t s);
void gemm_bf16_set_variant(int v);

// AllReduce point: out = own + sum_k peers[k] (float32 accumulation in order),
// followed by the full block's dropout + residual tail when `tail` has a
// residual (bf16 only)
// dense bf16 MFMA throughput probe: `workgroups` x 4 waves, each issuing
// 4 * iters v_mfma_f32_32x32x16_bf16; out holds workgroups * 256 floats
hipError_t mfma_probe(int workgroups, int iters, float *out, hipStream_t s);
// form 0: several 16-byte vectors per thread in flight (fastest alone); 1:
// one vector per thread with all inputs in flight and few registers, so the
// sum's waves fit on CUs beside a GEMM workgroup's (bf16, up to 7 peers).
// Both give the same bits.
hipError_t allreduce_point(bool bf16, const void *own, const void *peers, int64_t peer_stride,
                           int n_peers, void *out, int64_t n, hipStream_t s,
                           const DropRes *tail = nullptr, int form = 0);
// the form to use for a sum that runs beside compute kernels or alone (the
// process setting of oases_sum_variant, else that choice)
int allreduce_form(bool beside_compute);

// ---- full transformer block (bf16) ----
// z = LayerNorm(x) * w + b per row of x [rows, h] (biased variance, eps)
hipError_t layer_norm_fwd(const void *x, const void *w, const void *b, void *z, int rows, int h, float eps,
                          hipStream_t s);
// dx = g + LayerNorm backward of dz at x (weight w), and the column partials
// of sum_rows dz * xhat and sum_rows dz (fixed row chunks).  stats: 2*rows
// floats; partial: layer_norm_partial_floats(rows, h) floats.
hipError_t layer_norm_bwd(const void *dz, const void *x, const void *w, const void *g, void *dx,
                          float *stats, float *partial, int rows, int h, float eps, hipStream_t s);
// the LayerNorm weight gradients from those partials, in chunk order:
// dw (+)= sum_rows dz * xhat, db (+)= sum_rows dz (beta: accumulate)
hipError_t layer_norm_wgrad(const float *partial, float *dw, float *db, int rows, int h, int beta,
                            hipStream_t s);
int64_t layer_norm_partial_floats(int rows, int h);
// out = dropout backward of g (the mask and scale of `t`), n elements
hipError_t dropout_bwd(const void *g, void *out, int64_t n, const DropRes &t, hipStream_t s);
// largest grid (workgroups) of the AllReduce-point kernel
void allreduce_set_grid_cap(int cap);
// form of the AllReduce-point kernel for this process: 0 automatic, 1 always
// several vectors per thread, 2 always one vector per thread
void allreduce_set_variant(int v);
// workgroups that run an AllReduce point of nvec 8-element vectors fused into
// a GEMM launch (a multiple of 8, at most half the grid cap)
int allreduce_fused_wgs(int64_t nvec);

// db (+)= column sums of x[rows, cols] in a fixed order; partial needs
// colsum_partial_floats(rows, cols) floats.
int64_t colsum_partial_floats(int rows, int cols);
hipError_t colsum(bool bf16, const void *x, int rows, int cols, int ldx, float *partial, float *db,
                  int beta, hipStream_t s);

// Row stride of the lse / delta arrays: s rounded up to 64.
int attn_lse_stride(int s);
// 0 automatic; 1, 2, 3: OWN 1, 4, 2; 4, 5: OWN 1, 2 with tile pairs (tests, tuning)
void attention_set_variant(int v);

// Causal attention over QKV [nb*s, 3a] (columns [Q | K | V], head-major):
// O [nb*s, a], lse [nb, nh, attn_lse_stride(s)] (natural log).  bf16, d in {64, 128}.
hipError_t attention_fwd(int nb, int s, int nh, int d, int causal, const void *qkv, void *o,
                         float *lse, hipStream_t st);
// Backward: writes dQKV [nb*s, 3a].  Scratch: delta [nb, nh, attn_lse_stride(s)]
// floats (rowsum(dO * O)) and dsm, attn_ds_elems(nb, nh, s) bf16 (the dS
// matrices [nb*nh, s_pad, s_pad] passed from the dK/dV to the dQ kernel).
int64_t attn_ds_elems(int nb, int nh, int s);
hipError_t attention_bwd(int nb, int s, int nh, int d, int causal, const void *qkv,
                         const void *o, const void *dout, const float *lse, float *delta,
                         void *dsm, void *dqkv, hipStream_t st);

// ---- host-side entry helpers (executor.cpp) ----
// record the message of a failing context-free call (oases_last_call_error);
// returns code
int call_fail(int code, const std::string &msg);
// scratch of the attention backward: delta, then the dS matrices (256-byte aligned)
size_t attention_bwd_scratch_bytes(int nb, int s, int nh);
// argument checks of the attention backward (no HIP call); *need = scratch
// bytes, 0 for an empty problem
int attention_bwd_validate(int nb, int s, int nh, int d, int causal, const void *qkv, const void *o,
                           const void *dout, const float *lse, void *dqkv, size_t *need);
// validated attention backward on caller scratch; an oases_status, with the
// message of a failure kept for oases_last_call_error()
int attention_bwd_call(int nb, int s, int nh, int d, int causal, const void *qkv, const void *o,
                       const void *dout, const float *lse, void *dqkv, void *scratch, size_t scratch_bytes,
                       hipStream_t st);

}  // namespace oases
