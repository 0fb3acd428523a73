/*
 * oases_shard.h -- C ABI of liboases_shard: one GPU's tensor-model-parallel
 * (TMP) shard of a stack of attention / FFN blocks, run through the
 * overlapped training schedule with fine-grained recomputation of
 * "Oases: Efficient Large-Scale Model Training on Commodity Servers via
 * Overlapped and Automated Tensor Model Parallelism" (arXiv 2305.16121),
 * Section IV.
 *
 * Block l (a Megatron-style shard):
 *   attention: QKV = X W_in^T + b_in      (W_in [3a, h], columns [Q | K | V],
 *                                          each head-major, a = n_s * d)
 *              O   = causal softmax(Q K^T / sqrt(d)) V      per (sequence, head)
 *              P   = O W_out^T            (W_out [h, a])
 *   FFN:       U = X W_in^T + b_in,  H = gelu(U) = U * Phi(U)   (W_in [f_s, h])
 *              P = H W_out^T              (W_out [h, f_s])
 *   AllReduce point C(F):  Y = P + sum_{k=1}^{w-1} peer_k   (Section IV: the
 *              AllReduce output is the sum of its w inputs).  On one GPU the
 *              w-1 peer partials are caller-provided resident buffers that
 *              stand in for the other ranks.  Accumulated in float32 in the
 *              order own, peer_1, ..., peer_{w-1}; rounded once to the
 *              storage type (bf16: round to nearest even).
 *   X_{l+1} = Y_l.  Backward: dP = dY (Eq. (1): the gradient of each
 *              AllReduce input equals the gradient of its output), and the
 *              backward AllReduce point C(B) sums this shard's dX with the
 *              w-1 backward peer partials.
 *
 * Schedules (Section IV, Fig. 4, Algorithm 1): the batch is split along its
 * batch dimension into two sub-batches (rows [0, T_sb) and [T_sb, 2 T_sb) of
 * every [B*s, h] tensor, T_sb = (B/2) s).  Only block inputs are stored
 * between forward and backward (checkpoints); the backward of block l and
 * sub-batch sb is R (recompute from the stored input; the row GEMM is not
 * re-run and C(R) is not issued), B_dX, C(B) (started asynchronously),
 * B_dW.  Weight gradients: sub-batch 0 writes, sub-batch 1 accumulates.
 *
 * Conventions
 *  - All tensors are row-major and dense.  Token row r = b*s + t.
 *  - Storage type: float32 (OASES_F32) or bf16 (OASES_BF16) for activations,
 *    weights and biases; weight and bias gradients are always float32.
 *    Accumulation is float32 throughout.
 *  - Pointers are device pointers, 16-byte aligned, owned by the caller.  The
 *    library never allocates or frees device memory; it owns only HIP events
 *    and graphs it creates.  Streams are borrowed (hipStream_t as void*).
 *  - Every call returns an oases_status; nothing aborts or throws across the
 *    ABI.  On failure oases_last_error() holds a message.  Argument checks run
 *    before any HIP call, so a call that fails validation enqueues nothing.
 *  - All enqueueing calls are asynchronous on the bound streams; only
 *    oases_sync blocks the host.  One context belongs to one host thread.
 */
#ifndef OASES_SHARD_H
#define OASES_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oases_ctx oases_ctx; /* opaque; created by oases_create */

typedef enum {
  OASES_OK = 0,
  OASES_E_ARG = -1,         /* bad argument: null pointer, index out of range */
  OASES_E_STATE = -2,       /* call out of order (e.g. backward before forward) */
  OASES_E_SHAPE = -3,       /* configuration the kernels do not support */
  OASES_E_ALIGN = -4,       /* pointer not 16-byte aligned */
  OASES_E_HIP = -5,         /* a HIP runtime call failed; see oases_last_error */
  OASES_E_UNSUPPORTED = -6  /* valid request that this build does not implement */
} oases_status;

typedef enum { OASES_F32 = 0, OASES_BF16 = 1 } oases_dtype;
typedef enum { OASES_ATTN = 0, OASES_FFN = 1 } oases_block;

/* Step schedules (Section IV, Fig. 4).  OVERLAP_FINE issues every AllReduce
 * point on the side stream so that one sub-batch's sum overlaps the other
 * sub-batch's compute, ordered with events; OVERLAP_FUSED (same op list)
 * runs each AllReduce point on extra workgroups of the next GEMM launched on
 * the compute stream -- the other sub-batch's GEMM, or the dW GEMM of the
 * backward -- so the two run concurrently without cross-queue events
 * (float32 configurations issue the sum as its own kernel on the compute
 * stream).  The SERIAL modes issue everything on the compute stream.
 * DEFAULT_RECOMPUTE recomputes the whole block including its row GEMM and
 * issues C(R) (its result is discarded); NO_RECOMPUTE keeps every block's
 * intermediates from the forward pass (needs a larger workspace).
 * OVERLAP_STREAMS issues the same op list with one stream per sub-batch:
 * sub-batch 0's compute and AllReduce points on the compute stream,
 * sub-batch 1's on the side stream, so each sub-batch's sums and kernels run
 * beside the other's; the only cross-stream edges order the two
 * sub-batches' weight-gradient accumulation (and a fork and join per step),
 * except in the cool-down: from 64 MiB of AllReduce-point inputs
 * (T_sb * h * w elements) up, sub-batch 1's last weight gradients (B_dW of
 * layer 0) run on the compute stream, after sub-batch 0's, so that they
 * overlap sub-batch 1's dX GEMM and its last AllReduce point
 * (oases_schedule_ops reports that stream).
 * All modes give bit-identical results. */
typedef enum {
  OASES_OVERLAP_FINE = 0,
  OASES_SERIAL_FINE = 1,
  OASES_SERIAL_DEFAULT_RECOMPUTE = 2,
  OASES_SERIAL_NO_RECOMPUTE = 3,
  OASES_OVERLAP_FUSED = 4,
  OASES_OVERLAP_STREAMS = 5
} oases_mode;

/* Shape of the shard.  Constraints (OASES_E_SHAPE otherwise):
 *   n_layers in [1, 64]; blocks[l] in {OASES_ATTN, OASES_FFN};
 *   micro_batch >= 2 and even; seq >= 1;
 *   hidden, ffn_shard multiples of 64; tmp_width >= 1;
 *   attention blocks: head_dim in {64, 128}, heads_per_shard >= 1,
 *   and dtype OASES_BF16 (float32 attention is OASES_E_UNSUPPORTED);
 *   causal in {0, 1}.  The blocks array is copied by oases_create.
 * Full transformer block (the replicated tail F_j of Section IV; bf16 only,
 * OASES_E_UNSUPPORTED for float32): with full_block = 1 every block's column
 * GEMM reads LayerNorm(x) (weights ln_w, ln_b, epsilon ln_eps > 0; biased
 * variance) instead of its input x, and its AllReduce point yields
 * x + dropout(sum) instead of the sum.  Dropout drops each element with
 * probability drop_q / 65536 (drop_q in [0, 65535]): element e of a
 * sub-batch's [T_sb, h] tensor is kept iff word e % 4 of Philox4x64-10 at
 * counter (e / 4, sub_batch, 0, 0) under key (drop_seed, layer) is below
 * (65536 - drop_q) * 2^48, and kept elements are scaled by
 * 65536 / (65536 - drop_q).  gelu_tanh = 1 uses the tanh form of GeLU in the
 * FFN blocks (bf16 only). */
typedef struct {
  int32_t n_layers;
  const int32_t *blocks;
  int32_t micro_batch, seq, hidden;
  int32_t heads_per_shard, head_dim, ffn_shard, tmp_width;
  int32_t dtype;   /* oases_dtype */
  int32_t causal;
  int32_t full_block;  /* 0: bare blocks; 1: LayerNorm / dropout / residual */
  int32_t drop_q;
  uint64_t drop_seed;
  float ln_eps;
  int32_t gelu_tanh;
} oases_config;

/* Per-layer parameters.  N_in = 3a (attention) or f_s (FFN); N_mid = a or f_s.
 *   w_in [N_in, h], b_in [N_in], w_out [h, N_mid]           storage type
 *   dw_in [N_in, h], db_in [N_in], dw_out [h, N_mid]         float32, written
 *   (overwritten by sub-batch 0, accumulated by sub-batch 1 of each step).
 *   ln_w, ln_b [h] (storage type) and dln_w, dln_b [h] (float32, written the
 *   same way): the LayerNorm of full blocks; NULL otherwise. */
typedef struct {
  const void *w_in, *b_in, *w_out;
  void *dw_in, *db_in, *dw_out;
  const void *ln_w, *ln_b;
  void *dln_w, *dln_b;
} oases_layer_params;

/* Activation buffers (storage type unless stated):
 *   x   [B*s, h]   input of layer 0 (read only)
 *   y   [B*s, h]   output of the top layer (written by its C(F))
 *   dy  [B*s, h]   upstream gradient dL/dy (read only)
 *   dx  [B*s, h]   gradient w.r.t. x (written by layer 0's C(B))
 *   ckpt [L-1, B*s, h]  stored inputs of layers 1..L-1 (the only tensors kept
 *        between forward and backward); may be NULL when L == 1
 *   peers_fwd, peers_bwd [L, 2, w-1, T_sb, h]  resident peer partials of the
 *        forward and backward AllReduce points, indexed [layer][sub-batch][k];
 *        may be NULL when w == 1
 *   workspace: device scratch of at least oases_workspace_bytes(cfg, mode)
 *        bytes for every mode that will be run; 256-byte aligned. */
typedef struct {
  const void *x;
  void *y;
  const void *dy;
  void *dx;
  void *ckpt;
  const void *peers_fwd, *peers_bwd;
  void *workspace;
  size_t workspace_bytes;
} oases_buffers;

/* Validate cfg and create a context.  Makes no HIP call. */
int oases_create(const oases_config *cfg, oases_ctx **out);

/* Workspace bytes needed by `mode` (NO_RECOMPUTE needs per-layer
 * intermediates, the other modes one set per sub-batch).  No HIP call. */
int oases_workspace_bytes(const oases_config *cfg, int32_t mode, size_t *bytes);

/* Bind caller buffers and per_layer[n_layers] parameters.  Checks non-null
 * and 16-byte alignment of every pointer that the configuration needs.
 * Resets the per-step state.  No HIP call. */
int oases_bind(oases_ctx *c, const oases_buffers *b, const oases_layer_params *per_layer);

/* Borrow the compute stream and the side (communication) stream; NULL means
 * the default stream.  Passing the same stream twice serialises everything.
 * Creates the context's HIP events on the current device. */
int oases_set_streams(oases_ctx *c, void *compute_stream, void *side_stream);

/* Forward operator of block `layer` for sub-batch `sub_batch` (0 or 1):
 * the computation operator F_i followed by StartAsync of its communication
 * operator C_i(F) (Section IV: the forward sequence (F_i, C_i(F), F_j) and the
 * executor's StartAsync / Sync of Algorithm 1).  F runs on the compute stream
 * (after a Sync on the C(F) that produced its input), then C(F) -- the sum of
 * the shard's partial output and the w-1 peer partials -- on the side stream.
 * Requires layer_fwd of (layer-1, sub_batch) earlier in the step.  Only the
 * block input is kept (checkpoint); intermediates are not.
 * Errors (nothing is enqueued): OASES_E_ARG for layer / sub_batch out of
 * range, OASES_E_STATE if called out of order, before oases_bind /
 * oases_set_streams, or twice in one step; OASES_E_HIP if a launch fails. */
int layer_fwd(oases_ctx *c, int32_t layer, int32_t sub_batch);

/* Fine-grained backward of block `layer`, sub-batch `sub_batch` (Section IV,
 * Fig. 4d and Eq. (1)): R (recompute from the stored input, started after
 * the forward's communication operator, so no row GEMM and no C(R): by
 * Eq. (1) the AllReduce inputs' gradient is dY itself), then B_dX after a
 * Sync on the C(B) of (layer+1, sub_batch), StartAsync of C(B) on the side
 * stream, then B_dW on the compute stream.  Requires layer_fwd of the top
 * layer for this sub-batch and layer_bwd_recompute of (layer+1, sub_batch);
 * sub-batch 1 of a layer requires sub-batch 0 of the same layer first
 * (gradient accumulation order).  Errors as layer_fwd (OASES_E_STATE for
 * these orderings). */
int layer_bwd_recompute(oases_ctx *c, int32_t layer, int32_t sub_batch);

/* One whole step (forward + backward of every layer and both sub-batches) in
 * `mode` (Section IV, Algorithm 1: split the batch into two sub-batches, run
 * the forward with each sub-batch's AllReduce points overlapping the other's
 * compute, then the backward in fine-grained recompute order).  use_graph != 0
 * captures the step into a hipGraph on its first call per mode (needs a
 * non-default compute stream) and replays it afterwards.  Errors: OASES_E_ARG
 * for a bad mode or a workspace too small for it; OASES_E_STATE before
 * oases_bind / oases_set_streams; OASES_E_HIP if a launch or the capture
 * fails.  Nothing is enqueued on a validation error. */
int schedule_step(oases_ctx *c, int32_t mode, int32_t use_graph);

/* Op list of `mode` as issued by schedule_step, four int32 per op:
 * kind (0 F, 1 C_F, 2 R, 3 C_R, 4 B_dX, 5 C_B, 6 B_dW), layer, sub-batch,
 * stream (0 compute, 1 side).  Writes at most `cap` ops, returns the count in
 * *n_ops.  No HIP call. */
int oases_schedule_ops(const oases_ctx *c, int32_t mode, int32_t *ops, int32_t cap,
                       int32_t *n_ops);

/* Block the host until both bound streams are idle. */
int oases_sync(oases_ctx *c);

/* Last error message of the context ("" if none); valid until the next call. */
const char *oases_last_error(const oases_ctx *c);

/* Release events and graphs.  Safe on NULL. */
void oases_destroy(oases_ctx *c);

/* Timing instrumentation of one kernel class (0 GEMM forward/recompute,
 * 1 GEMM data gradient, 2 GEMM weight gradient, 3 attention forward,
 * 4 attention backward, 5 AllReduce-point sum, 6 bias-gradient column sum).
 * After oases_profile_begin, every eager (not graph-captured) launch of that
 * class, for at most max_launches launches, is timed by a pair of HIP events
 * carried in the dispatch packets of its kernels (hipExtLaunchKernelGGL):
 * from the start of its first kernel to the end of its last, on the stream
 * it is launched on.  oases_profile_end waits for those events and returns
 * the summed time and the number of launches timed.  Timing state is per
 * host thread.  kernel_class 7 times every class.
 * oases_profile_timeline ends a timing run like oases_profile_end but
 * returns each timed launch: its class, its stream (0 the compute stream,
 * 1 the side stream, 2 another) and the start and end of its kernels in ms
 * after the start of the first timed launch (all streams share the GPU's
 * clock), in launch order.  classes, streams, start_ms and end_ms are caller
 * arrays of cap entries; more timed launches than cap is OASES_E_ARG (the
 * run stays open).  Blocks the host until the timed launches have ended. */
int oases_profile_begin(oases_ctx *c, int32_t kernel_class, int32_t max_launches);
int oases_profile_end(oases_ctx *c, double *total_ms, int32_t *launches);
int oases_profile_timeline(oases_ctx *c, int32_t cap, int32_t *classes, int32_t *streams, double *start_ms,
                           double *end_ms, int32_t *launches);

/* ---- single-kernel entry points (used by tests and the benchmark) ----
 * They run one kernel family on `stream` (NULL = default) with the same
 * device code as the step, so each kernel can be checked and timed alone. */

/* Dense bf16 matrix-core throughput probe (a measurement aid, not a step of
 * the path): `workgroups` workgroups of 4 waves, each wave issuing
 * 4 * iters independent v_mfma_f32_32x32x16_bf16 (32*32*16*2 FLOP each) on
 * register operands.  out: caller device buffer of workgroups * 256 floats
 * (16-byte aligned), overwritten with per-lane checksums.  1 <= workgroups
 * <= 65536 and iters >= 1, else OASES_E_ARG.  Asynchronous on `stream`. */
int oases_mfma_probe(int32_t workgroups, int32_t iters, float *out, void *stream);

/* AllReduce-point sum (Section IV): out[i] = own[i] + sum_k peers[k*peer_stride + i]
 * for i < n, float32 accumulation in that order, one rounding to dtype.
 * n_peers >= 0; n a multiple of 8. */
int oases_allreduce_point(int32_t dtype, const void *own, const void *peers, int64_t peer_stride,
                          int32_t n_peers, void *out, int64_t n, void *stream);

/* General GEMM of the path: C[M,N] = sum_k A(m,k) B(k,n), float32 accumulation.
 *   a_layout 0: A stored [M][lda] (k contiguous);  1: A stored [K][lda] (m contiguous)
 *   b_layout 0: B stored [N][ldb] (k contiguous);  1: B stored [K][ldb] (n contiguous)
 *   epilogue 0: C = acc;  1: C = acc + bias[n];  2: C = gelu(acc + bias[n]) and, if pre
 *            != NULL, pre = acc + bias[n];  3: C = acc * gelu'(aux[m][n]);
 *            4: C (float32) = acc, plus the old C when beta != 0;
 *            5 (bfloat16 only): as 4, and pre (float32, m elements) = the sums of
 *            A(m, k) over k, plus the old pre when beta != 0 (a bias gradient
 *            taken beside its weight gradient); 6, 7 (bfloat16 only): as 2 and 3
 *            with the tanh form of GeLU.
 * Supported: layouts (0,0) with epilogues 0-2 and 6 (forward / recompute),
 * (0,1) with 0, 3 and 7 (data gradient), (1,1) with 4 and 5 (weight
 * gradient).  Storage-type
 * operands; the contiguous dimension of every operand and N are multiples of
 * 8; leading dimensions in elements, multiples of 8.  pre and C (epilogues
 * 0-3) use ldc; aux uses ld_aux. */
int oases_gemm(int32_t dtype, int32_t a_layout, int32_t b_layout, int32_t epilogue, int32_t m,
               int32_t n, int32_t k, const void *a, int32_t lda, const void *b, int32_t ldb,
               void *c, int32_t ldc, const void *bias, void *pre, const void *aux, int32_t ld_aux,
               int32_t beta, void *stream);

/* Tile configuration of the bf16 GEMMs for this process: 0 = automatic (the
 * default), 1..22 force one of the compiled tile shapes and pipeline depths
 * (tests and tuning sweeps; 20..22 split each tile's k loop between two wave
 * groups, or run their tile with one group where the k-tile count is odd).  Returns OASES_E_ARG for other values. */
int oases_gemm_tile_variant(int32_t variant);

/* Largest number of workgroups of the AllReduce-point sum kernel for this
 * process (default 512); a sum fused into a GEMM launch (OVERLAP_FUSED)
 * uses at most half as many.  A smaller grid leaves CUs to the compute that
 * runs beside a sum.  Graphs already captured keep the value they were
 * captured with.  1..65536, else OASES_E_ARG. */
int oases_sum_grid_cap(int32_t workgroups);

/* Form of the AllReduce-point sum kernel for this process.  Form A keeps the
 * loads of several 16-byte vectors per thread in flight (fastest alone);
 * form B takes one vector per thread with all w inputs in flight, in few
 * enough registers that its waves fit on a CU beside a GEMM workgroup's, so
 * a sum issued beside the other sub-batch's compute shares CUs with it
 * instead of taking them.  0 = automatic (the default: form B for the sums
 * of the overlapped schedules, form A for sums that run alone and for
 * oases_allreduce_point), 1 = always form A, 2 = always form B.  Both add in
 * the same order and give the same bits.  Graphs already captured keep the
 * form they were captured with.  OASES_E_ARG for other values. */
int oases_sum_variant(int32_t variant);

/* Attention work split for this process.  A workgroup has 4 waves of 32
 * rows each; OWN of them own distinct row tiles (sharing each staged block)
 * and 4/OWN split the walk over the other operand.  With tile pairs a
 * workgroup takes two row tiles, one with a long and one with a short causal
 * walk.  0 = automatic (the default: for the causal forward with d = 128,
 * variant 9 when it gives at least 128 workgroups; otherwise for the
 * forward 8-wave workgroups with the largest OWN in {4, 2} (or 1 for
 * d = 64) that gives 256 workgroups, else the largest OWN of 4 waves that
 * does; for the backward,
 * OWN 1 with pairs when pairs alone give 256 workgroups of a causal
 * attention, else as the 4-wave forward), 1 = OWN 1, 2 = OWN 4, 3 = OWN 2,
 * 4 = OWN 1 with pairs, 5 = OWN 2 with pairs; 6, 7, 8: the forward with
 * 8-wave workgroups and OWN 2, 4, 1 (OWN 1 for d = 64 only; d = 128 runs
 * OWN 2), 9: the forward with 8-wave workgroups whose two owned tiles are a
 * long and a short causal walk; for 6 to 9 the backward is automatic.  For
 * tests and tuning; OASES_E_ARG for other values. */
int oases_attention_variant(int32_t variant);

/* Causal (causal = 1) or full attention forward over QKV [nb*s, 3a]
 * (columns [Q | K | V], each head-major) -> O [nb*s, a] and the per-row
 * log-sum-exp lse [nb, n_h, s_pad] (float32, natural log, row stride
 * s_pad = s rounded up to a multiple of 64).  bf16 only; d in {64, 128}. */
int oases_attention_fwd(int32_t nb, int32_t s, int32_t n_h, int32_t d, int32_t causal,
                        const void *qkv, void *o, float *lse, void *stream);

/* Attention backward of the attention block (Section IV: the backward B of
 * the attention operator of an F_i; the softmax probabilities are rebuilt
 * from lse, nothing of the forward beyond O and lse is kept).  Inputs: QKV
 * [nb*s, 3a] as in oases_attention_fwd, O and dO [nb*s, a] (bf16), lse
 * [nb, n_h, s_pad] (float32, as oases_attention_fwd writes it).  Output:
 * dQKV [nb*s, 3a] (bf16; columns [dQ | dK | dV], head-major), fully written.
 * workspace: caller-owned device scratch of at least
 * oases_attention_bwd_workspace_bytes(nb, s, n_h) bytes (delta =
 * rowsum(dO * O) per query, then the dS matrices [nb*n_h, s_pad, s_pad] in
 * bf16 that the dK/dV kernel passes to the dQ kernel); it needs no
 * initialisation and is overwritten.  d in {64, 128}; 16-byte aligned
 * pointers.  Errors (before any launch; message in oases_last_call_error):
 * OASES_E_ARG, OASES_E_ALIGN; OASES_E_HIP if a launch fails.  Asynchronous on
 * `stream`. */
int oases_attention_bwd_workspace_bytes(int32_t nb, int32_t s, int32_t n_h, size_t *bytes);
int oases_attention_bwd(int32_t nb, int32_t s, int32_t n_h, int32_t d, int32_t causal, const void *qkv,
                        const void *o, const void *dout, const float *lse, void *dqkv, void *workspace,
                        size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * oases_attention_bwd with its scratch in a static device array of 48 MiB
 * instead of a workspace argument.  Each GPU the library runs on holds its
 * own copy of the array until the process ends; the call allocates nothing.
 * Arguments, layouts and outputs as oases_attention_bwd.  A problem whose
 * scratch (oases_attention_bwd_workspace_bytes) exceeds 48 MiB is rejected
 * with OASES_E_ARG before any launch (message in oases_last_call_error).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams or threads) race and give wrong results; calls ordered
 * on one stream are safe.  Nothing in the array needs to start at zero: each
 * call writes every entry it reads. */
int oases_attention_bwd_noalloc(int32_t nb, int32_t s, int32_t n_h, int32_t d, int32_t causal,
                                const void *qkv, const void *o, const void *dout, const float *lse,
                                void *dqkv, void *stream);

/* Message of the last failing call on this thread that takes no context
 * (oases_create and the single-kernel entry points); "" if none. */
const char *oases_last_call_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OASES_SHARD_H */
