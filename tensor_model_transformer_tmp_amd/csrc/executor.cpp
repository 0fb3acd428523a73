// liboases_shard: context, validation, workspace layout, the op lists of the
// four step schedules and their issue on a compute and a side HIP stream,
// hipGraph capture, and the C-ABI entry points.
//
// Schedule source: "Oases: Efficient Large-Scale Model Training on Commodity
// Servers via Overlapped and Automated Tensor Model Parallelism"
// (arXiv 2305.16121), Section IV: the batch split into two sub-batches whose
// operators pipeline (Fig. 4b); fine-grained recomputation that starts after
// the forward communication operator and drops C(R) (Eq. (1), Fig. 4d); the
// runtime executor whose computation operators have Forward / Recompute /
// Backward and whose communication operators have StartAsync / Sync, storing
// only the input of each recompute sequence (Algorithm 1).  StartAsync here is
// "record an event on the compute stream, make the side stream wait on it,
// launch the AllReduce-point kernel on the side stream, record its event";
// Sync is "make the compute stream wait on that event".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/oases_shard.h"
#include "kernels.h"

using namespace oases;

namespace oases {
LaunchTimer &launch_timer() {
  static thread_local LaunchTimer t;
  return t;
}
}  // namespace oases

namespace {

enum OpKind : int32_t { OP_F = 0, OP_CF = 1, OP_R = 2, OP_CR = 3, OP_BDX = 4, OP_CB = 5, OP_BDW = 6 };
struct Op {
  int32_t kind, layer, sb, stream;
};

// kernel classes for timing instrumentation
enum KClass : int32_t {
  KC_GEMM_FWD = 0, KC_GEMM_DX = 1, KC_GEMM_DW = 2, KC_ATTN_FWD = 3, KC_ATTN_BWD = 4,
  KC_SUM = 5, KC_COLSUM = 6, KC_COUNT = 7
};

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

struct Dims {
  int L, B, s, h, ns, d, fs, w, dtype, causal;
  bool full;          // LayerNorm / dropout / residual around every block
  int drop_q, tanh;   // dropout probability in 1/65536; tanh-form GeLU
  uint64_t drop_seed;
  float eps;
  int T, a, nb;  // tokens per sub-batch, attention width, sequences per sub-batch
  size_t esz;
  bool any_attn, any_ffn;
  std::vector<int32_t> blocks;
  int n_in(int l) const { return blocks[l] == OASES_ATTN ? 3 * a : fs; }
  int n_mid(int l) const { return blocks[l] == OASES_ATTN ? a : fs; }
  int max_n_in() const { return std::max(any_attn ? 3 * a : 0, any_ffn ? fs : 0); }
};

// workspace layout for one mode (byte offsets)
struct WsLayout {
  size_t P[2], dxo[2], dpre[2], dO[2], delta[2];
  size_t ads[2];  // attention backward: the dS matrices passed from the dK/dV to the dQ kernel
  size_t act_bytes;      // one activation slot
  size_t act0;           // first slot; slot (i, sb) at act0 + (i*2 + sb) * act_bytes
  int n_slots;
  // offsets inside a slot
  size_t s_U, s_H, s_QKV, s_O, s_LSE;
  size_t colsum[2];  // per sub-batch: the sub-batches' column sums may run concurrently
  size_t s_Z;                     // full blocks: LayerNorm output in a slot
  size_t dS[2], dZ[2], lnst[2];   // full blocks: dropout backward, C(B) sum, row statistics
  size_t lnpart[2];               // full blocks: LayerNorm weight-gradient partials
  size_t gbuf[2];
  size_t cr_out;
  size_t total;
};

WsLayout make_layout(const Dims &D, int mode) {
  WsLayout o{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t r = off; off = align_up(off + bytes); return r; };
  const size_t th = (size_t)D.T * D.h * D.esz;
  const size_t lse_bytes = (size_t)D.nb * D.ns * attn_lse_stride(D.s) * sizeof(float);
  for (int sb = 0; sb < 2; ++sb) {
    o.P[sb] = take(th);
    o.dxo[sb] = take(th);
    o.dpre[sb] = take((size_t)D.T * D.max_n_in() * D.esz);
    o.dO[sb] = D.any_attn ? take((size_t)D.T * D.a * D.esz) : 0;
    o.delta[sb] = D.any_attn ? take(lse_bytes) : 0;
    o.ads[sb] = D.any_attn ? take((size_t)attn_ds_elems(D.nb, D.ns, D.s) * 2) : 0;
    o.dS[sb] = D.full ? take(th) : 0;
    o.dZ[sb] = D.full ? take(th) : 0;
    o.lnst[sb] = D.full ? take((size_t)D.T * 2 * sizeof(float)) : 0;
  }
  for (int sb = 0; sb < 2; ++sb)
    o.lnpart[sb] = D.full ? take((size_t)layer_norm_partial_floats(D.T, D.h) * sizeof(float)) : 0;
  // activation slot: FFN {U, H} or attention {QKV, O, LSE}; slot size is the max
  size_t ffn_sz = 0, attn_sz = 0;
  if (D.any_ffn) ffn_sz = 2 * align_up((size_t)D.T * D.fs * D.esz);
  if (D.any_attn)
    attn_sz = align_up((size_t)D.T * 3 * D.a * D.esz) + align_up((size_t)D.T * D.a * D.esz) +
              align_up(lse_bytes);
  o.act_bytes = align_up(std::max(ffn_sz, attn_sz)) + (D.full ? align_up(th) : 0);
  o.s_Z = align_up(std::max(ffn_sz, attn_sz));
  o.s_U = 0;
  o.s_H = D.any_ffn ? align_up((size_t)D.T * D.fs * D.esz) : 0;
  o.s_QKV = 0;
  o.s_O = D.any_attn ? align_up((size_t)D.T * 3 * D.a * D.esz) : 0;
  o.s_LSE = D.any_attn ? o.s_O + align_up((size_t)D.T * D.a * D.esz) : 0;
  o.n_slots = (mode == OASES_SERIAL_NO_RECOMPUTE) ? D.L : 1;
  o.act0 = take(o.act_bytes * 2 * o.n_slots);
  for (int sb = 0; sb < 2; ++sb) o.colsum[sb] = take((size_t)colsum_partial_floats(D.T, D.max_n_in()) * sizeof(float));
  if (D.L > 1) {
    o.gbuf[0] = take((size_t)2 * th);
    o.gbuf[1] = take((size_t)2 * th);
  }
  o.cr_out = (mode == OASES_SERIAL_DEFAULT_RECOMPUTE) ? take(th) : 0;
  o.total = off;
  return o;
}

int check_config(const oases_config *cfg, Dims *D, std::string *err) {
  auto fail = [&](int code, const char *msg) { if (err) *err = msg; return code; };
  if (!cfg) return fail(OASES_E_ARG, "config is NULL");
  if (cfg->n_layers < 1 || cfg->n_layers > 64) return fail(OASES_E_SHAPE, "n_layers must be in [1, 64]");
  if (!cfg->blocks) return fail(OASES_E_ARG, "blocks is NULL");
  if (cfg->dtype != OASES_F32 && cfg->dtype != OASES_BF16) return fail(OASES_E_ARG, "bad dtype");
  if (cfg->micro_batch < 2 || cfg->micro_batch % 2) return fail(OASES_E_SHAPE, "micro_batch must be even and >= 2");
  if (cfg->seq < 1) return fail(OASES_E_SHAPE, "seq must be >= 1");
  if (cfg->hidden < 64 || cfg->hidden % 64) return fail(OASES_E_SHAPE, "hidden must be a positive multiple of 64");
  if (cfg->tmp_width < 1) return fail(OASES_E_SHAPE, "tmp_width must be >= 1");
  if (cfg->causal != 0 && cfg->causal != 1) return fail(OASES_E_ARG, "causal must be 0 or 1");
  Dims d{};
  d.L = cfg->n_layers;
  d.blocks.assign(cfg->blocks, cfg->blocks + cfg->n_layers);
  for (int32_t b : d.blocks) {
    if (b == OASES_ATTN) d.any_attn = true;
    else if (b == OASES_FFN) d.any_ffn = true;
    else return fail(OASES_E_ARG, "block kind must be OASES_ATTN or OASES_FFN");
  }
  if (d.any_ffn && (cfg->ffn_shard < 64 || cfg->ffn_shard % 64))
    return fail(OASES_E_SHAPE, "ffn_shard must be a positive multiple of 64");
  if (d.any_attn) {
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return fail(OASES_E_SHAPE, "head_dim must be 64 or 128");
    if (cfg->heads_per_shard < 1) return fail(OASES_E_SHAPE, "heads_per_shard must be >= 1");
    if (cfg->dtype != OASES_BF16) return fail(OASES_E_UNSUPPORTED, "attention blocks need bf16 storage");
  }
  const int64_t T = (int64_t)(cfg->micro_batch / 2) * cfg->seq;
  if (T * (int64_t)cfg->hidden >= (int64_t(1) << 31) || T * 3LL * cfg->heads_per_shard * cfg->head_dim >= (int64_t(1) << 31) ||
      T * (int64_t)cfg->ffn_shard >= (int64_t(1) << 31))
    return fail(OASES_E_SHAPE, "a sub-batch tensor exceeds 2^31 elements");
  d.B = cfg->micro_batch; d.s = cfg->seq; d.h = cfg->hidden;
  d.ns = d.any_attn ? cfg->heads_per_shard : 0;
  d.d = d.any_attn ? cfg->head_dim : 0;
  d.fs = d.any_ffn ? cfg->ffn_shard : 0;
  d.w = cfg->tmp_width; d.dtype = cfg->dtype; d.causal = cfg->causal;
  d.T = (int)T; d.a = d.ns * d.d; d.nb = d.B / 2;
  d.esz = cfg->dtype == OASES_BF16 ? 2 : 4;
  if (cfg->full_block != 0 && cfg->full_block != 1) return fail(OASES_E_ARG, "full_block must be 0 or 1");
  if (cfg->gelu_tanh != 0 && cfg->gelu_tanh != 1) return fail(OASES_E_ARG, "gelu_tanh must be 0 or 1");
  if ((cfg->full_block || cfg->gelu_tanh) && cfg->dtype != OASES_BF16)
    return fail(OASES_E_UNSUPPORTED, "full blocks and tanh GeLU need bf16 storage");
  if (cfg->full_block && (cfg->drop_q < 0 || cfg->drop_q > 65535))
    return fail(OASES_E_ARG, "drop_q must be in [0, 65535]");
  if (cfg->full_block && !(cfg->ln_eps > 0.f)) return fail(OASES_E_ARG, "ln_eps must be > 0");
  d.full = cfg->full_block == 1;
  d.drop_q = d.full ? cfg->drop_q : 0;
  d.drop_seed = cfg->drop_seed;
  d.eps = cfg->ln_eps;
  d.tanh = cfg->gelu_tanh;
  if (D) *D = std::move(d);
  return OASES_OK;
}

// OVERLAP_STREAMS cool-down (Exec::cooldown): sub-batch 1's last weight
// gradients move to sub-batch 0's stream when the step's last AllReduce point
// outlasts the cross-queue wait the move puts on the step's critical path.
// Measured: the 4096- and 8192-hidden pairs (128 and 256 MiB of sum inputs)
// 1% faster, the 1024-hidden pair (16 MiB) 2% slower.
bool cooldown_move(const Dims &d) { return (int64_t)d.T * d.h * d.w * (int64_t)d.esz >= ((int64_t)64 << 20); }

std::vector<Op> build_ops(int L, int mode, bool cool) {
  std::vector<Op> ops;
  const int side = (mode == OASES_OVERLAP_FINE || mode == OASES_OVERLAP_FUSED) ? 1 : 0;
  const bool by_sb = mode == OASES_OVERLAP_STREAMS;  // stream = sub-batch
  for (int l = 0; l < L; ++l)
    for (int sb = 0; sb < 2; ++sb) {
      ops.push_back({OP_F, l, sb, by_sb ? sb : 0});
      ops.push_back({OP_CF, l, sb, by_sb ? sb : side});
    }
  for (int l = L - 1; l >= 0; --l)
    for (int sb = 0; sb < 2; ++sb) {
      if (mode != OASES_SERIAL_NO_RECOMPUTE) ops.push_back({OP_R, l, sb, by_sb ? sb : 0});
      if (mode == OASES_SERIAL_DEFAULT_RECOMPUTE) ops.push_back({OP_CR, l, sb, 0});
      ops.push_back({OP_BDX, l, sb, by_sb ? sb : 0});
      ops.push_back({OP_CB, l, sb, by_sb ? sb : side});
      ops.push_back({OP_BDW, l, sb, by_sb ? (cool && l == 0 ? 0 : sb) : 0});
    }
  return ops;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// message of the last failing context-free call on this thread
thread_local std::string g_call_err;

}  // namespace

namespace oases {

int call_fail(int code, const std::string &msg) {
  g_call_err = msg;
  return code;
}

size_t attention_bwd_scratch_bytes(int nb, int s, int nh) {
  return align_up((size_t)nb * nh * attn_lse_stride(s) * sizeof(float)) + (size_t)attn_ds_elems(nb, nh, s) * 2;
}

int attention_bwd_validate(int nb, int s, int nh, int d, int causal, const void *qkv, const void *o,
                           const void *dout, const float *lse, void *dqkv, size_t *need) {
  *need = 0;
  if (nb < 0 || s < 0 || nh < 0 || (d != 64 && d != 128) || (causal != 0 && causal != 1))
    return call_fail(OASES_E_ARG, "attention backward: need nb, s, n_h >= 0, d in {64, 128}, causal in {0, 1}");
  if ((int64_t)nb * s * 3 * nh * d > ((int64_t)1 << 31) || s > (1 << 20))
    return call_fail(OASES_E_ARG, "attention backward: qkv larger than 2^31 elements or s > 2^20");
  if (nb == 0 || s == 0 || nh == 0) return OASES_OK;
  if (!qkv || !o || !dout || !lse || !dqkv) return call_fail(OASES_E_ARG, "attention backward: a pointer is NULL");
  if (!aligned16(qkv) || !aligned16(o) || !aligned16(dout) || !aligned16(lse) || !aligned16(dqkv))
    return call_fail(OASES_E_ALIGN, "attention backward: a pointer is not 16-byte aligned");
  *need = attention_bwd_scratch_bytes(nb, s, nh);
  return OASES_OK;
}

int attention_bwd_call(int nb, int s, int nh, int d, int causal, const void *qkv, const void *o,
                       const void *dout, const float *lse, void *dqkv, void *scratch, size_t scratch_bytes,
                       hipStream_t st) {
  size_t need = 0;
  if (int r = attention_bwd_validate(nb, s, nh, d, causal, qkv, o, dout, lse, dqkv, &need)) return r;
  if (need == 0) return OASES_OK;  // empty problem
  if (!scratch) return call_fail(OASES_E_ARG, "attention backward: scratch is NULL");
  if (!aligned16(scratch)) return call_fail(OASES_E_ALIGN, "attention backward: scratch is not 16-byte aligned");
  if (scratch_bytes < need)
    return call_fail(OASES_E_ARG, "attention backward: scratch of " + std::to_string(scratch_bytes) +
                                      " bytes, need " + std::to_string(need));
  float *delta = static_cast<float *>(scratch);
  void *dsm = static_cast<char *>(scratch) + align_up((size_t)nb * nh * attn_lse_stride(s) * sizeof(float));
  const hipError_t e = attention_bwd(nb, s, nh, d, causal, qkv, o, dout, lse, delta, dsm, dqkv, st);
  if (e != hipSuccess) return call_fail(OASES_E_HIP, std::string("attention backward: ") + hipGetErrorString(e));
  return OASES_OK;
}

}  // namespace oases

struct oases_ctx {
  Dims D;
  bool bound = false;
  oases_buffers buf{};
  std::vector<oases_layer_params> prm;
  hipStream_t cs = nullptr, ss = nullptr;
  bool streams_set = false;
  std::vector<hipEvent_t> evF, evCF, evBdX, evCB;
  // OVERLAP_STREAMS: sub-batch 0's dW_in and db_in of layer l done [l], its
  // LayerNorm weight gradients done [L + l], fork (after sub-batch 0's first
  // column GEMM) [2L], join [2L + 1], its dW_out of layer l done [2L + 2 + l];
  // cool-down: sub-batch 1's layer-0 dW_out operands ready [3L + 2], its
  // layer-0 dX GEMM done [3L + 3]
  std::vector<hipEvent_t> evSB;
  hipGraphExec_t gexec[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  std::vector<uint8_t> fwd_done, bwd_done;
  std::string err;
  // timing instrumentation
  int prof_class = -1;  // KC_COUNT: every class
  std::vector<hipEvent_t> prof_ev;
  std::vector<int32_t> prof_cls;  // class of each timed launch (event pair)
  std::vector<int32_t> prof_str;  // its stream: 0 compute, 1 side, 2 other
  size_t prof_used = 0;
  bool capturing = false;
};

namespace {

int set_err(oases_ctx *c, int code, const std::string &msg) {
  if (c) c->err = msg;
  return code;
}

#define HIPX(expr)                                                                      \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return set_err(c, OASES_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

void destroy_graphs(oases_ctx *c) {
  for (auto &g : c->gexec)
    if (g) { (void)hipGraphExecDestroy(g); g = nullptr; }
}

// ---- the executor: one op at a time --------------------------------------

struct Exec {
  oases_ctx *c;
  const WsLayout &W;
  int mode;
  bool overlap;  // side stream distinct from the compute stream
  // OVERLAP_STREAMS: every op of sub-batch 1 (compute and its AllReduce
  // points) on the side stream, of sub-batch 0 on the compute stream
  bool by_sb = false;
  hipStream_t cst(int sb) const { return by_sb && sb == 1 ? c->ss : c->cs; }
  // OVERLAP_STREAMS cool-down: sub-batch 1's B_dW of layer 0 runs on sub-batch
  // 0's stream, which has issued all of its own work by then.  dW_out runs
  // beside sub-batch 1's dX GEMM, dW_in beside its last AllReduce point
  // (instead of all three after one another on one stream), and both follow
  // sub-batch 0's weight gradients on that stream, the accumulation order.
  bool cooldown(int l, int sb) const { return by_sb && l == 0 && sb == 1 && cooldown_move(D()); }
  // OVERLAP_FUSED (bf16): an AllReduce point waits here and runs as extra
  // workgroups of the next GEMM launched on the compute stream
  bool fused = false;
  FusedSum pending{};

  char *ws() const { return static_cast<char *>(c->buf.workspace); }
  const Dims &D() const { return c->D; }
  size_t th_bytes() const { return (size_t)D().T * D().h * D().esz; }
  bool bf16() const { return D().dtype == OASES_BF16; }

  const char *layer_in(int l, int sb) const {
    const char *base = l == 0 ? static_cast<const char *>(c->buf.x)
                              : static_cast<const char *>(c->buf.ckpt) + (size_t)(l - 1) * 2 * th_bytes();
    return base + sb * th_bytes();
  }
  char *layer_out(int l, int sb) const {
    char *base = l == D().L - 1 ? static_cast<char *>(c->buf.y)
                                : static_cast<char *>(c->buf.ckpt) + (size_t)l * 2 * th_bytes();
    return base + sb * th_bytes();
  }
  // gradient w.r.t. the output of layer l (read by its backward)
  const char *grad_out(int l, int sb) const {
    const char *base = l == D().L - 1 ? static_cast<const char *>(c->buf.dy) : ws() + W.gbuf[l % 2];
    return base + sb * th_bytes();
  }
  // gradient w.r.t. the input of layer l (written by its C(B))
  char *grad_in(int l, int sb) const {
    char *base = l == 0 ? static_cast<char *>(c->buf.dx) : ws() + W.gbuf[(l - 1) % 2];
    return base + sb * th_bytes();
  }
  char *slot(int l, int sb) const {
    const int i = W.n_slots == 1 ? 0 : l;
    return ws() + W.act0 + (size_t)(i * 2 + sb) * W.act_bytes;
  }
  // the column GEMM's input: the block input, or (full blocks) its LayerNorm
  const char *gemm_in(int l, int sb) const { return D().full ? slot(l, sb) + W.s_Z : layer_in(l, sb); }
  // the full block's dropout + residual after block l's AllReduce point
  DropRes tail(int l, int sb) const {
    const Dims &d = D();
    DropRes t{};
    t.res = layer_in(l, sb);
    t.seed = d.drop_seed;
    t.layer = (uint64_t)l;
    t.sb = (uint64_t)sb;
    t.drop = d.drop_q > 0;
    t.thr = t.drop ? (uint64_t)(65536 - d.drop_q) << 48 : 0;
    t.scale = t.drop ? 65536.f / (float)(65536 - d.drop_q) : 1.f;
    return t;
  }
  const char *peers(const void *p, int l, int sb) const {
    const size_t per = (size_t)(D().w - 1) * th_bytes();
    return static_cast<const char *>(p) + (size_t)(l * 2 + sb) * per;
  }

  // Time one launch of kernel class `cls`: arm the next event pair, which the
  // kernels launched until prof_end carry in their dispatch packets.
  bool profiled(int cls) const {
    return (c->prof_class == cls || c->prof_class == KC_COUNT) && !c->capturing;
  }
  int prof_begin(int cls, hipStream_t) {
    if (!profiled(cls)) return OASES_OK;
    if (c->prof_used + 2 > c->prof_ev.size()) return OASES_OK;  // ring full: stop timing
    launch_timer() = LaunchTimer{c->prof_ev[c->prof_used], c->prof_ev[c->prof_used + 1]};
    return OASES_OK;
  }
  int prof_end(int cls, hipStream_t s) {
    if (!profiled(cls)) return OASES_OK;
    const bool launched = launch_timer().stop && !launch_timer().start;  // a kernel took the pair
    launch_timer() = LaunchTimer{};
    if (launched) {
      c->prof_cls[c->prof_used / 2] = cls;
      c->prof_str[c->prof_used / 2] = s == c->cs ? 0 : (s == c->ss ? 1 : 2);
      c->prof_used += 2;
    }
    return OASES_OK;
  }

  int gemm(int cls, oases::Layout la, oases::Layout lb, Epi epi, const GemmArgs &g, hipStream_t s);
  // an AllReduce point, optionally with the full block's tail (t.res set);
  // may_fuse: the sum may wait for the next GEMM launch (fused overlap)
  int sum(const void *own, const void *pr, void *out, hipStream_t s, const DropRes &t = DropRes{},
          bool may_fuse = true) {
    if (fused && may_fuse) {  // deferred to the next GEMM launch (flush_pending at the latest)
      const int64_t n = (int64_t)D().T * D().h;
      pending = FusedSum{own, pr, n, out, n / 8, D().w - 1, allreduce_fused_wgs(n / 8), t};
      return OASES_OK;
    }
    if (int r = prof_begin(KC_SUM, s)) return r;
    // a sum issued beside the other sub-batch's compute (side stream, or a
    // stream per sub-batch) takes the low-register form that shares CUs
    const int form = allreduce_form(overlap || by_sb);
    HIPX(allreduce_point(bf16(), own, pr, (int64_t)D().T * D().h, D().w - 1, out, (int64_t)D().T * D().h, s, &t,
                         form));
    return prof_end(KC_SUM, s);
  }

  // a deferred sum with no GEMM after it runs as its own kernel
  int flush_pending() {
    if (!pending.wgs) return OASES_OK;
    const FusedSum f = pending;
    pending = FusedSum{};
    return sum(f.own, f.peers, f.out, c->cs, f.tail, false);
  }

  // gradient w.r.t. the partial sums of block l's AllReduce point (Eq. (1)):
  // dY itself, or (full blocks) its dropout backward
  const void *dP(int l, int sb) const { return D().full ? static_cast<const void *>(ws() + W.dS[sb]) : grad_out(l, sb); }

  // column part of block l (F or R): writes the slot's activations.
  // OVERLAP_STREAMS: sub-batch 1 starts once sub-batch 0's first column
  // GEMM is done (the fork event), so the two chains run half a phase apart
  // as in the schedule's pipeline: one sub-batch's AllReduce point meets the
  // other's GEMMs.  Started together, the two identical chains reach their
  // AllReduce points at the same time and the sums run beside each other
  // (measured on MI355X at the 8192-hidden pair: 3.47 -> 3.36 ms per step,
  // sums beside compute 0.65 -> 0.80; lagging by a whole block compute, or
  // by the column part with attention, gained little).
  int start_lag(int l, int sb) {
    if (by_sb && l == 0 && sb == 0) HIPX(hipEventRecord(c->evSB[2 * D().L], cst(sb)));
    return OASES_OK;
  }

  int column_part(int l, int sb, bool keep_pre) {
    const Dims &d = D();
    const oases_layer_params &p = c->prm[l];
    char *sl = slot(l, sb);
    if (d.full) HIPX(layer_norm_fwd(layer_in(l, sb), p.ln_w, p.ln_b, sl + W.s_Z, d.T, d.h, d.eps, cst(sb)));
    const void *x = gemm_in(l, sb);
    if (d.blocks[l] == OASES_FFN) {
      GemmArgs g{};
      g.M = d.T; g.N = d.fs; g.K = d.h;
      g.A = x; g.lda = d.h; g.B = p.w_in; g.ldb = d.h;
      g.C = sl + W.s_H; g.ldc = d.fs; g.bias = p.b_in;
      g.pre = keep_pre ? sl + W.s_U : nullptr; g.ld_pre = d.fs;
      if (int r = gemm(KC_GEMM_FWD, KC, KC, d.tanh ? EPI_BIAS_GELU_TANH : EPI_BIAS_GELU, g, cst(sb))) return r;
      return start_lag(l, sb);
    }
    GemmArgs g{};
    g.M = d.T; g.N = 3 * d.a; g.K = d.h;
    g.A = x; g.lda = d.h; g.B = p.w_in; g.ldb = d.h;
    g.C = sl + W.s_QKV; g.ldc = 3 * d.a; g.bias = p.b_in;
    if (int r = gemm(KC_GEMM_FWD, KC, KC, EPI_BIAS, g, cst(sb))) return r;
    if (int r = start_lag(l, sb)) return r;
    if (int r = prof_begin(KC_ATTN_FWD, cst(sb))) return r;
    HIPX(attention_fwd(d.nb, d.s, d.ns, d.d, d.causal, sl + W.s_QKV, sl + W.s_O,
                       reinterpret_cast<float *>(sl + W.s_LSE), cst(sb)));
    return prof_end(KC_ATTN_FWD, cst(sb));
  }

  // row-parallel GEMM of block l: partial P[sb] = act W_out^T
  int row_part(int l, int sb) {
    const Dims &d = D();
    const oases_layer_params &p = c->prm[l];
    char *sl = slot(l, sb);
    GemmArgs g{};
    g.M = d.T; g.N = d.h; g.K = d.n_mid(l);
    g.A = d.blocks[l] == OASES_FFN ? sl + W.s_H : sl + W.s_O; g.lda = d.n_mid(l);
    g.B = p.w_out; g.ldb = d.n_mid(l);
    g.C = ws() + W.P[sb]; g.ldc = d.h;
    return gemm(KC_GEMM_FWD, KC, KC, EPI_STORE, g, cst(sb));
  }

  int op_F(int l, int sb) {
    if (overlap && l > 0) HIPX(hipStreamWaitEvent(cst(sb), c->evCF[(l - 1) * 2 + sb], 0));
    if (by_sb && l == 0 && sb == 1) HIPX(hipStreamWaitEvent(c->ss, c->evSB[2 * D().L], 0));  // the fork
    const bool keep = mode == OASES_SERIAL_NO_RECOMPUTE;
    if (int r = column_part(l, sb, keep)) return r;
    if (int r = row_part(l, sb)) return r;
    if (overlap) HIPX(hipEventRecord(c->evF[l * 2 + sb], cst(sb)));
    return OASES_OK;
  }
  int op_CF(int l, int sb) {
    hipStream_t s = overlap ? c->ss : cst(sb);
    if (overlap) HIPX(hipStreamWaitEvent(s, c->evF[l * 2 + sb], 0));
    if (int r = sum(ws() + W.P[sb], D().w > 1 ? peers(c->buf.peers_fwd, l, sb) : nullptr,
                    layer_out(l, sb), s, D().full ? tail(l, sb) : DropRes{}))
      return r;
    if (overlap) HIPX(hipEventRecord(c->evCF[l * 2 + sb], s));
    return OASES_OK;
  }
  int op_R(int l, int sb) {
    if (int r = column_part(l, sb, true)) return r;
    if (mode == OASES_SERIAL_DEFAULT_RECOMPUTE) return row_part(l, sb);
    return OASES_OK;
  }
  int op_CR(int l, int sb) {
    return sum(ws() + W.P[sb], D().w > 1 ? peers(c->buf.peers_fwd, l, sb) : nullptr, ws() + W.cr_out, cst(sb),
               D().full ? tail(l, sb) : DropRes{});
  }
  int op_BdX(int l, int sb) {
    const Dims &d = D();
    const oases_layer_params &p = c->prm[l];
    if (overlap && l < d.L - 1) HIPX(hipStreamWaitEvent(cst(sb), c->evCB[(l + 1) * 2 + sb], 0));
    char *sl = slot(l, sb);
    const void *dy = dP(l, sb);
    if (d.full)  // the AllReduce inputs' gradient: dropout backward of dY (Eq. (1))
      HIPX(dropout_bwd(grad_out(l, sb), ws() + W.dS[sb], (int64_t)d.T * d.h, tail(l, sb), cst(sb)));
    if (cooldown(l, sb)) HIPX(hipEventRecord(c->evSB[3 * d.L + 2], cst(sb)));  // dY and R's activations
    char *dpre = ws() + W.dpre[sb];
    if (d.blocks[l] == OASES_FFN) {
      GemmArgs g{};  // dU = (dY W_out) * gelu'(U)
      g.M = d.T; g.N = d.fs; g.K = d.h;
      g.A = dy; g.lda = d.h; g.B = p.w_out; g.ldb = d.fs;
      g.C = dpre; g.ldc = d.fs; g.aux = sl + W.s_U; g.ld_aux = d.fs;
      if (int r = gemm(KC_GEMM_DX, KC, MC, d.tanh ? EPI_GELU_BWD_TANH : EPI_GELU_BWD, g, cst(sb))) return r;
    } else {
      GemmArgs g{};  // dO = dY W_o
      g.M = d.T; g.N = d.a; g.K = d.h;
      g.A = dy; g.lda = d.h; g.B = p.w_out; g.ldb = d.a;
      g.C = ws() + W.dO[sb]; g.ldc = d.a;
      if (int r = gemm(KC_GEMM_DX, KC, MC, EPI_STORE, g, cst(sb))) return r;
      if (int r = prof_begin(KC_ATTN_BWD, cst(sb))) return r;
      HIPX(attention_bwd(d.nb, d.s, d.ns, d.d, d.causal, sl + W.s_QKV, sl + W.s_O, ws() + W.dO[sb],
                         reinterpret_cast<const float *>(sl + W.s_LSE),
                         reinterpret_cast<float *>(ws() + W.delta[sb]), ws() + W.ads[sb], dpre, cst(sb)));
      if (int r = prof_end(KC_ATTN_BWD, cst(sb))) return r;
    }
    GemmArgs g{};  // dX_own = dpre W_in
    g.M = d.T; g.N = d.h; g.K = d.n_in(l);
    g.A = dpre; g.lda = d.n_in(l); g.B = p.w_in; g.ldb = d.h;
    g.C = ws() + W.dxo[sb]; g.ldc = d.h;
    if (int r = gemm(KC_GEMM_DX, KC, MC, EPI_STORE, g, cst(sb))) return r;
    if (overlap) HIPX(hipEventRecord(c->evBdX[l * 2 + sb], cst(sb)));
    if (cooldown(l, sb)) HIPX(hipEventRecord(c->evSB[3 * d.L + 3], cst(sb)));  // dpre and dX_own
    return OASES_OK;
  }
  int op_CB(int l, int sb) {
    const Dims &d = D();
    hipStream_t s = overlap ? c->ss : cst(sb);
    if (overlap) HIPX(hipStreamWaitEvent(s, c->evBdX[l * 2 + sb], 0));
    if (!d.full) {
      if (int r = sum(ws() + W.dxo[sb], d.w > 1 ? peers(c->buf.peers_bwd, l, sb) : nullptr, grad_in(l, sb), s))
        return r;
    } else {  // the sum (never deferred: its LayerNorm backward follows at once), then
      // dX = dY + LayerNorm backward of the sum, and the LayerNorm weight gradients
      if (int r = sum(ws() + W.dxo[sb], d.w > 1 ? peers(c->buf.peers_bwd, l, sb) : nullptr, ws() + W.dZ[sb], s,
                      DropRes{}, false))
        return r;
      const oases_layer_params &p = c->prm[l];
      float *part = reinterpret_cast<float *>(ws() + W.lnpart[sb]);
      HIPX(layer_norm_bwd(ws() + W.dZ[sb], layer_in(l, sb), p.ln_w, grad_out(l, sb), grad_in(l, sb),
                          reinterpret_cast<float *>(ws() + W.lnst[sb]), part, d.T, d.h, d.eps, s));
      // the sub-batches' LayerNorm weight gradients accumulate in a fixed
      // order; with a stream per sub-batch only this last launch waits
      if (by_sb && sb == 1) HIPX(hipStreamWaitEvent(s, c->evSB[d.L + l], 0));
      HIPX(layer_norm_wgrad(part, static_cast<float *>(p.dln_w), static_cast<float *>(p.dln_b), d.T, d.h, sb, s));
      if (by_sb && sb == 0) HIPX(hipEventRecord(c->evSB[d.L + l], s));
    }
    if (overlap) HIPX(hipEventRecord(c->evCB[l * 2 + sb], s));
    return OASES_OK;
  }
  int op_BdW(int l, int sb) {
    // the two sub-batches' weight gradients accumulate in a fixed order, one
    // GEMM at a time (see weight_grads)
    if (int r = weight_grads(l, sb)) return r;
    if (by_sb && sb == 0) HIPX(hipEventRecord(c->evSB[l], c->cs));
    return OASES_OK;
  }
  int weight_grads(int l, int sb) {
    const Dims &d = D();
    const oases_layer_params &p = c->prm[l];
    char *sl = slot(l, sb);
    const void *dy = dP(l, sb);
    const char *dpre = ws() + W.dpre[sb];
    const int nmid = d.n_mid(l), nin = d.n_in(l);
    GemmArgs g{};  // dW_out[h, nmid] (+)= dY^T act
    g.M = d.h; g.N = nmid; g.K = d.T;
    g.A = dy; g.lda = d.h;
    g.B = d.blocks[l] == OASES_FFN ? sl + W.s_H : sl + W.s_O; g.ldb = nmid;
    g.C = p.dw_out; g.ldc = nmid; g.beta = sb;
    // with a stream per sub-batch, sub-batch 1 adds into each weight gradient
    // once sub-batch 0 has written it: its dW_out GEMM waits for sub-batch 0's
    // dW_out only, and so runs beside sub-batch 0's dW_in GEMM.  In the
    // cool-down both GEMMs follow sub-batch 0's on its stream, and wait for
    // their operands from sub-batch 1's stream instead.
    const int L = d.L;
    const bool cool = cooldown(l, sb);
    hipStream_t s = cool ? c->cs : cst(sb);
    if (cool) HIPX(hipStreamWaitEvent(s, c->evSB[3 * L + 2], 0));
    else if (by_sb && sb == 1) HIPX(hipStreamWaitEvent(s, c->evSB[2 * L + 2 + l], 0));
    if (int r = gemm(KC_GEMM_DW, MC, MC, EPI_F32, g, s)) return r;
    if (by_sb && sb == 0) HIPX(hipEventRecord(c->evSB[2 * L + 2 + l], c->cs));
    if (cool) HIPX(hipStreamWaitEvent(s, c->evSB[3 * L + 3], 0));  // dpre
    else if (by_sb && sb == 1) HIPX(hipStreamWaitEvent(s, c->evSB[l], 0));  // dW_in and db_in
    GemmArgs g2{};  // dW_in[nin, h] (+)= dpre^T X
    g2.M = nin; g2.N = d.h; g2.K = d.T;
    g2.A = dpre; g2.lda = nin; g2.B = gemm_in(l, sb); g2.ldb = d.h;
    g2.C = p.dw_in; g2.ldc = d.h; g2.beta = sb;
    if (bf16()) {  // db_in (+)= column sums of dpre, computed by the same GEMM
      g2.colsum = static_cast<float *>(p.db_in);
      return gemm(KC_GEMM_DW, MC, MC, EPI_F32, g2, s);
    }
    if (int r = gemm(KC_GEMM_DW, MC, MC, EPI_F32, g2, s)) return r;
    if (int r = prof_begin(KC_COLSUM, s)) return r;
    HIPX(colsum(bf16(), dpre, d.T, nin, nin, reinterpret_cast<float *>(ws() + W.colsum[sb]),
                static_cast<float *>(p.db_in), sb, s));
    return prof_end(KC_COLSUM, s);
  }

  int run(const Op &o) {
    switch (o.kind) {
      case OP_F: return op_F(o.layer, o.sb);
      case OP_CF: return op_CF(o.layer, o.sb);
      case OP_R: return op_R(o.layer, o.sb);
      case OP_CR: return op_CR(o.layer, o.sb);
      case OP_BDX: return op_BdX(o.layer, o.sb);
      case OP_CB: return op_CB(o.layer, o.sb);
      case OP_BDW: return op_BdW(o.layer, o.sb);
    }
    return set_err(c, OASES_E_ARG, "bad op");
  }
};

int Exec::gemm(int cls, oases::Layout la, oases::Layout lb, Epi epi, const GemmArgs &g0, hipStream_t s) {
  GemmArgs g = g0;
  if (fused && pending.wgs && s == c->cs && g.M > 0 && g.N > 0) {
    g.sum = pending;
    pending = FusedSum{};
  }
  if (int r = prof_begin(cls, s)) return r;
  if (bf16()) HIPX(gemm_bf16(la, lb, epi, g, s));
  else HIPX(gemm_f32(la, lb, epi, g, s));
  return prof_end(cls, s);
}

int ensure_events(oases_ctx *c) {
  if (!c->evF.empty()) return OASES_OK;
  const int n = c->D.L * 2;
  c->evSB.resize(n + 4 + c->D.L, nullptr);
  for (auto *v : {&c->evF, &c->evCF, &c->evBdX, &c->evCB, &c->evSB}) {
    if (v != &c->evSB) v->resize(n, nullptr);
    // device-internal ordering only: no timing, no system-scope fence
    for (auto &e : *v) HIPX(hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence));
  }
  return OASES_OK;
}

int need_ready(oases_ctx *c, int mode) {
  if (!c->bound) return set_err(c, OASES_E_STATE, "buffers are not bound");
  if (!c->streams_set) return set_err(c, OASES_E_STATE, "streams are not set");
  const WsLayout W = make_layout(c->D, mode);
  if (c->buf.workspace_bytes < W.total)
    return set_err(c, OASES_E_ARG, "workspace too small for this mode: need " + std::to_string(W.total) +
                                       " bytes");
  return OASES_OK;
}

int issue_ops(oases_ctx *c, int mode, const std::vector<Op> &ops) {
  const WsLayout W = make_layout(c->D, mode);
  Exec ex{c, W, mode, mode == OASES_OVERLAP_FINE && c->ss != c->cs};
  ex.fused = mode == OASES_OVERLAP_FUSED && c->D.dtype == OASES_BF16;
  ex.by_sb = mode == OASES_OVERLAP_STREAMS && c->ss != c->cs;
  const int L = c->D.L;
  // OVERLAP_STREAMS fork: the side stream (sub-batch 1) starts after sub-batch
  // 0's first column GEMM on the compute stream, and so after what precedes
  // the step there (start_lag, op_F)
  for (const Op &o : ops)
    if (int r = ex.run(o)) return r;
  if (int r = ex.flush_pending()) return r;
  if (ex.overlap) {  // join the side stream into the compute stream
    HIPX(hipStreamWaitEvent(c->cs, c->evCB[0 * 2 + 1], 0));
  }
  if (ex.by_sb) {  // join
    HIPX(hipEventRecord(c->evSB[2 * L + 1], c->ss));
    HIPX(hipStreamWaitEvent(c->cs, c->evSB[2 * L + 1], 0));
  }
  return OASES_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int oases_create(const oases_config *cfg, oases_ctx **out) {
  if (!out) return OASES_E_ARG;
  *out = nullptr;
  Dims d;
  std::string err;
  const int r = check_config(cfg, &d, &err);
  if (r) return call_fail(r, "oases_create: " + err);
  oases_ctx *c = new oases_ctx();
  c->D = std::move(d);
  c->fwd_done.assign(c->D.L * 2, 0);
  c->bwd_done.assign(c->D.L * 2, 0);
  *out = c;
  return OASES_OK;
}

int oases_workspace_bytes(const oases_config *cfg, int32_t mode, size_t *bytes) {
  if (!bytes) return OASES_E_ARG;
  if (mode < 0 || mode > 5) return OASES_E_ARG;
  Dims d;
  if (int r = check_config(cfg, &d, nullptr)) return r;
  *bytes = make_layout(d, mode).total;
  return OASES_OK;
}

int oases_bind(oases_ctx *c, const oases_buffers *b, const oases_layer_params *per_layer) {
  if (!c) return OASES_E_ARG;
  if (!b || !per_layer) return set_err(c, OASES_E_ARG, "buffers or per_layer is NULL");
  const Dims &D = c->D;
  struct P { const void *p; const char *name; bool need; };
  const P ps[] = {{b->x, "x", true}, {b->y, "y", true}, {b->dy, "dy", true}, {b->dx, "dx", true},
                  {b->ckpt, "ckpt", D.L > 1}, {b->peers_fwd, "peers_fwd", D.w > 1},
                  {b->peers_bwd, "peers_bwd", D.w > 1}, {b->workspace, "workspace", true}};
  for (const P &p : ps) {
    if (!p.need) continue;
    if (!p.p) return set_err(c, OASES_E_ARG, std::string(p.name) + " is NULL");
    if (!aligned16(p.p)) return set_err(c, OASES_E_ALIGN, std::string(p.name) + " is not 16-byte aligned");
  }
  if ((uintptr_t)b->workspace % ALIGN) return set_err(c, OASES_E_ALIGN, "workspace is not 256-byte aligned");
  const size_t need = make_layout(D, OASES_SERIAL_FINE).total;
  if (b->workspace_bytes < need)
    return set_err(c, OASES_E_ARG, "workspace smaller than oases_workspace_bytes(OASES_SERIAL_FINE) = " +
                                       std::to_string(need));
  for (int l = 0; l < D.L; ++l) {
    const oases_layer_params &q = per_layer[l];
    const void *lp[] = {q.w_in, q.b_in, q.w_out, q.dw_in, q.db_in, q.dw_out, q.ln_w, q.ln_b, q.dln_w, q.dln_b};
    const char *nm[] = {"w_in", "b_in", "w_out", "dw_in", "db_in", "dw_out", "ln_w", "ln_b", "dln_w", "dln_b"};
    for (int i = 0; i < (D.full ? 10 : 6); ++i) {
      if (!lp[i]) return set_err(c, OASES_E_ARG, "layer " + std::to_string(l) + " " + nm[i] + " is NULL");
      if (!aligned16(lp[i]))
        return set_err(c, OASES_E_ALIGN, "layer " + std::to_string(l) + " " + nm[i] + " is not 16-byte aligned");
    }
  }
  destroy_graphs(c);
  c->buf = *b;
  c->prm.assign(per_layer, per_layer + D.L);
  c->bound = true;
  std::fill(c->fwd_done.begin(), c->fwd_done.end(), 0);
  std::fill(c->bwd_done.begin(), c->bwd_done.end(), 0);
  c->err.clear();
  return OASES_OK;
}

int oases_set_streams(oases_ctx *c, void *compute_stream, void *side_stream) {
  if (!c) return OASES_E_ARG;
  if (int r = ensure_events(c)) return r;
  destroy_graphs(c);
  c->cs = static_cast<hipStream_t>(compute_stream);
  c->ss = static_cast<hipStream_t>(side_stream);
  c->streams_set = true;
  return OASES_OK;
}

int layer_fwd(oases_ctx *c, int32_t layer, int32_t sub_batch) {
  if (!c) return OASES_E_ARG;
  if (layer < 0 || layer >= c->D.L) return set_err(c, OASES_E_ARG, "layer out of range");
  if (sub_batch != 0 && sub_batch != 1) return set_err(c, OASES_E_ARG, "sub_batch must be 0 or 1");
  if (!c->bound) return set_err(c, OASES_E_STATE, "buffers are not bound");
  if (layer == 0 && sub_batch == 0) {  // a new step starts
    std::fill(c->fwd_done.begin(), c->fwd_done.end(), 0);
    std::fill(c->bwd_done.begin(), c->bwd_done.end(), 0);
  }
  if (layer > 0 && !c->fwd_done[(layer - 1) * 2 + sub_batch])
    return set_err(c, OASES_E_STATE, "layer_fwd needs the previous layer's forward of this sub-batch");
  if (c->fwd_done[layer * 2 + sub_batch]) return set_err(c, OASES_E_STATE, "layer_fwd already issued in this step");
  if (int r = need_ready(c, OASES_SERIAL_FINE)) return r;
  const WsLayout W = make_layout(c->D, OASES_SERIAL_FINE);
  Exec ex{c, W, OASES_SERIAL_FINE, c->ss != c->cs};
  if (int r = ex.op_F(layer, sub_batch)) return r;
  if (int r = ex.op_CF(layer, sub_batch)) return r;
  c->fwd_done[layer * 2 + sub_batch] = 1;
  return OASES_OK;
}

int layer_bwd_recompute(oases_ctx *c, int32_t layer, int32_t sub_batch) {
  if (!c) return OASES_E_ARG;
  const int L = c->D.L;
  if (layer < 0 || layer >= L) return set_err(c, OASES_E_ARG, "layer out of range");
  if (sub_batch != 0 && sub_batch != 1) return set_err(c, OASES_E_ARG, "sub_batch must be 0 or 1");
  if (!c->bound) return set_err(c, OASES_E_STATE, "buffers are not bound");
  if (!c->fwd_done[(L - 1) * 2 + sub_batch])
    return set_err(c, OASES_E_STATE, "backward before the forward of this sub-batch finished");
  if (layer < L - 1 && !c->bwd_done[(layer + 1) * 2 + sub_batch])
    return set_err(c, OASES_E_STATE, "backward needs the layer above first");
  if (sub_batch == 1 && !c->bwd_done[layer * 2 + 0])
    return set_err(c, OASES_E_STATE, "sub-batch 1 of a layer needs sub-batch 0 first (gradient order)");
  if (c->bwd_done[layer * 2 + sub_batch]) return set_err(c, OASES_E_STATE, "backward already issued in this step");
  if (int r = need_ready(c, OASES_SERIAL_FINE)) return r;
  const WsLayout W = make_layout(c->D, OASES_SERIAL_FINE);
  Exec ex{c, W, OASES_SERIAL_FINE, c->ss != c->cs};
  if (int r = ex.op_R(layer, sub_batch)) return r;
  if (int r = ex.op_BdX(layer, sub_batch)) return r;
  if (int r = ex.op_CB(layer, sub_batch)) return r;
  if (int r = ex.op_BdW(layer, sub_batch)) return r;
  if (ex.overlap && layer == 0) HIPX(hipStreamWaitEvent(c->cs, c->evCB[sub_batch], 0));
  c->bwd_done[layer * 2 + sub_batch] = 1;
  return OASES_OK;
}

int schedule_step(oases_ctx *c, int32_t mode, int32_t use_graph) {
  if (!c) return OASES_E_ARG;
  if (mode < 0 || mode > 5) return set_err(c, OASES_E_ARG, "bad mode");
  if (int r = need_ready(c, mode)) return r;
  const std::vector<Op> ops = build_ops(c->D.L, mode, cooldown_move(c->D));
  std::fill(c->fwd_done.begin(), c->fwd_done.end(), 0);
  std::fill(c->bwd_done.begin(), c->bwd_done.end(), 0);
  if (!use_graph) return issue_ops(c, mode, ops);
  if (!c->gexec[mode]) {
    if (c->cs == nullptr) return set_err(c, OASES_E_ARG, "graph capture needs a non-default compute stream");
    HIPX(hipStreamBeginCapture(c->cs, hipStreamCaptureModeThreadLocal));
    c->capturing = true;
    const int r = issue_ops(c, mode, ops);
    c->capturing = false;
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(c->cs, &graph);
    if (r) { if (graph) (void)hipGraphDestroy(graph); return r; }
    if (e != hipSuccess) return set_err(c, OASES_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    const hipError_t e2 = hipGraphInstantiate(&c->gexec[mode], graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e2 != hipSuccess) {
      c->gexec[mode] = nullptr;
      return set_err(c, OASES_E_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e2));
    }
  }
  HIPX(hipGraphLaunch(c->gexec[mode], c->cs));
  return OASES_OK;
}

int oases_schedule_ops(const oases_ctx *c, int32_t mode, int32_t *ops, int32_t cap, int32_t *n_ops) {
  if (!c || !n_ops || (cap > 0 && !ops) || cap < 0) return OASES_E_ARG;
  if (mode < 0 || mode > 5) return OASES_E_ARG;
  const std::vector<Op> v = build_ops(c->D.L, mode, cooldown_move(c->D));
  *n_ops = (int32_t)v.size();
  for (int i = 0; i < (int)v.size() && i < cap; ++i) {
    ops[4 * i + 0] = v[i].kind; ops[4 * i + 1] = v[i].layer;
    ops[4 * i + 2] = v[i].sb; ops[4 * i + 3] = v[i].stream;
  }
  return OASES_OK;
}

int oases_sync(oases_ctx *c) {
  if (!c) return OASES_E_ARG;
  if (!c->streams_set) return set_err(c, OASES_E_STATE, "streams are not set");
  HIPX(hipStreamSynchronize(c->cs));
  if (c->ss != c->cs) HIPX(hipStreamSynchronize(c->ss));
  return OASES_OK;
}

const char *oases_last_error(const oases_ctx *c) { return c ? c->err.c_str() : "NULL context"; }

void oases_destroy(oases_ctx *c) {
  if (!c) return;
  destroy_graphs(c);
  for (auto *v : {&c->evF, &c->evCF, &c->evBdX, &c->evCB, &c->evSB, &c->prof_ev})
    for (auto &e : *v)
      if (e) (void)hipEventDestroy(e);
  delete c;
}

// ---- timing instrumentation ----

int oases_profile_begin(oases_ctx *c, int32_t kernel_class, int32_t max_launches) {
  if (!c) return OASES_E_ARG;
  if (kernel_class < 0 || kernel_class > KC_COUNT || max_launches < 1 || max_launches > 1 << 16)
    return set_err(c, OASES_E_ARG, "bad kernel class or launch count");
  for (auto &e : c->prof_ev) if (e) (void)hipEventDestroy(e);
  c->prof_ev.assign((size_t)max_launches * 2, nullptr);
  c->prof_cls.assign((size_t)max_launches, -1);
  c->prof_str.assign((size_t)max_launches, -1);
  for (auto &e : c->prof_ev) HIPX(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
  c->prof_used = 0;
  c->prof_class = kernel_class;
  launch_timer() = LaunchTimer{};
  return OASES_OK;
}

int oases_profile_end(oases_ctx *c, double *total_ms, int32_t *launches) {
  if (!c || !total_ms || !launches) return OASES_E_ARG;
  double tot = 0;
  for (size_t i = 0; i + 1 < c->prof_used; i += 2) {
    HIPX(hipEventSynchronize(c->prof_ev[i + 1]));
    float ms = 0;
    HIPX(hipEventElapsedTime(&ms, c->prof_ev[i], c->prof_ev[i + 1]));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int32_t)(c->prof_used / 2);
  c->prof_class = -1;
  c->prof_used = 0;
  launch_timer() = LaunchTimer{};
  return OASES_OK;
}

int oases_profile_timeline(oases_ctx *c, int32_t cap, int32_t *classes, int32_t *streams, double *start_ms,
                           double *end_ms, int32_t *launches) {
  if (!c || !launches || cap < 0 || (cap > 0 && (!classes || !streams || !start_ms || !end_ms)))
    return OASES_E_ARG;
  const size_t n = c->prof_used / 2;
  if (n > (size_t)cap) return set_err(c, OASES_E_ARG, "timeline buffers hold fewer launches than were timed");
  for (size_t i = 0; i < n; ++i) {
    HIPX(hipEventSynchronize(c->prof_ev[2 * i + 1]));
    float a = 0, b = 0;
    HIPX(hipEventElapsedTime(&a, c->prof_ev[0], c->prof_ev[2 * i]));
    HIPX(hipEventElapsedTime(&b, c->prof_ev[0], c->prof_ev[2 * i + 1]));
    classes[i] = c->prof_cls[i];
    streams[i] = c->prof_str[i];
    start_ms[i] = a;
    end_ms[i] = b;
  }
  *launches = (int32_t)n;
  c->prof_class = -1;
  c->prof_used = 0;
  launch_timer() = LaunchTimer{};
  return OASES_OK;
}

// ---- single-kernel entry points ----

int oases_mfma_probe(int32_t workgroups, int32_t iters, float *out, void *stream) {
  if (workgroups < 1 || workgroups > 1 << 16 || iters < 1 || !out) return OASES_E_ARG;
  if (!aligned16(out)) return OASES_E_ALIGN;
  return mfma_probe(workgroups, iters, out, static_cast<hipStream_t>(stream)) == hipSuccess ? OASES_OK
                                                                                          : OASES_E_HIP;
}

int oases_allreduce_point(int32_t dtype, const void *own, const void *peers, int64_t peer_stride,
                          int32_t n_peers, void *out, int64_t n, void *stream) {
  if (dtype != OASES_F32 && dtype != OASES_BF16) return OASES_E_ARG;
  if (n < 0 || n % 8 || n_peers < 0 || (n_peers > 0 && (!peers || peer_stride % 8))) return OASES_E_ARG;
  if (n == 0) return OASES_OK;
  if (!own || !out) return OASES_E_ARG;
  if (!aligned16(own) || !aligned16(out) || (n_peers > 0 && !aligned16(peers))) return OASES_E_ALIGN;
  const hipError_t e = allreduce_point(dtype == OASES_BF16, own, peers, peer_stride, n_peers, out, n,
                                       static_cast<hipStream_t>(stream), nullptr, allreduce_form(false));
  return e == hipSuccess ? OASES_OK : OASES_E_HIP;
}

int oases_gemm(int32_t dtype, int32_t a_layout, int32_t b_layout, int32_t epilogue, int32_t m,
               int32_t n, int32_t k, const void *a, int32_t lda, const void *b, int32_t ldb,
               void *c_, int32_t ldc, const void *bias, void *pre, const void *aux, int32_t ld_aux,
               int32_t beta, void *stream) {
  if (dtype != OASES_F32 && dtype != OASES_BF16) return OASES_E_ARG;
  if ((a_layout != 0 && a_layout != 1) || (b_layout != 0 && b_layout != 1)) return OASES_E_ARG;
  const bool fwd = a_layout == 0 && b_layout == 0, dx = a_layout == 0 && b_layout == 1,
             dw = a_layout == 1 && b_layout == 1;
  const bool tanh_epi = (epilogue == 6 || epilogue == 7) && dtype == OASES_BF16;
  if (!((fwd && ((epilogue >= 0 && epilogue <= 2) || (epilogue == 6 && tanh_epi))) ||
        (dx && (epilogue == 0 || epilogue == 3 || (epilogue == 7 && tanh_epi))) ||
        (dw && (epilogue == 4 || (epilogue == 5 && dtype == OASES_BF16)))))
    return OASES_E_UNSUPPORTED;
  if (m < 0 || n < 0 || k < 0 || n % 8) return OASES_E_ARG;
  if (m == 0 || n == 0) return OASES_OK;
  if (!a || !b || !c_) return OASES_E_ARG;
  if ((epilogue == 1 || epilogue == 2 || epilogue == 6) && !bias) return OASES_E_ARG;
  if ((epilogue == 3 || epilogue == 7) && (!aux || ld_aux < n || ld_aux % 8)) return OASES_E_ARG;
  if (epilogue == 5 && (!pre || ((uintptr_t)pre & 3))) return OASES_E_ARG;
  // contiguous dimension of each operand: A: k (layout 0) or m (1); B: k (0) or n (1)
  const int a_cont = a_layout == 0 ? k : m, a_rows = a_layout == 0 ? m : k;
  const int b_cont = b_layout == 0 ? k : n, b_rows = b_layout == 0 ? n : k;
  (void)a_rows; (void)b_rows;
  if (a_cont % 8 || b_cont % 8 || lda < a_cont || ldb < b_cont || ldc < n || lda % 8 || ldb % 8 ||
      ldc % 8)
    return OASES_E_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c_) || (pre && epilogue != 5 && !aligned16(pre)) ||
      (aux && !aligned16(aux)) || (bias && ((uintptr_t)bias & 7)))
    return OASES_E_ALIGN;
  GemmArgs g{};
  g.M = m; g.N = n; g.K = k; g.A = a; g.lda = lda; g.B = b; g.ldb = ldb; g.C = c_; g.ldc = ldc;
  g.bias = bias; g.pre = pre; g.ld_pre = ldc; g.aux = aux; g.ld_aux = ld_aux; g.beta = beta;
  const oases::Layout la = a_layout ? MC : KC, lb = b_layout ? MC : KC;
  if (epilogue == 5) { g.colsum = static_cast<float *>(pre); g.pre = nullptr; }
  const Epi epi = static_cast<Epi>(epilogue == 5 ? 4 : epilogue);
  const hipError_t e = dtype == OASES_BF16 ? gemm_bf16(la, lb, epi, g, static_cast<hipStream_t>(stream))
                                           : gemm_f32(la, lb, epi, g, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? OASES_OK : OASES_E_HIP;
}

int oases_sum_grid_cap(int32_t workgroups) {
  if (workgroups < 1 || workgroups > 65536) return OASES_E_ARG;
  allreduce_set_grid_cap(workgroups);
  return OASES_OK;
}

int oases_sum_variant(int32_t variant) {
  if (variant < 0 || variant > 2) return call_fail(OASES_E_ARG, "oases_sum_variant: 0, 1 or 2");
  allreduce_set_variant(variant);
  return OASES_OK;
}

int oases_attention_variant(int32_t variant) {
  if (variant < 0 || variant > 9) return OASES_E_ARG;
  attention_set_variant(variant);
  return OASES_OK;
}

int oases_gemm_tile_variant(int32_t variant) {
  if (variant < 0 || variant > 22) return OASES_E_ARG;
  gemm_bf16_set_variant(variant);
  return OASES_OK;
}

int oases_attention_fwd(int32_t nb, int32_t s, int32_t n_h, int32_t d, int32_t causal, const void *qkv,
                        void *o, float *lse, void *stream) {
  if (nb < 0 || s < 0 || n_h < 0 || (d != 64 && d != 128) || (causal != 0 && causal != 1)) return OASES_E_ARG;
  if (nb == 0 || s == 0 || n_h == 0) return OASES_OK;
  if (!qkv || !o || !lse) return OASES_E_ARG;
  if (!aligned16(qkv) || !aligned16(o) || !aligned16(lse)) return OASES_E_ALIGN;
  const hipError_t e = attention_fwd(nb, s, n_h, d, causal, qkv, o, lse, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? OASES_OK : OASES_E_HIP;
}

int oases_attention_bwd_workspace_bytes(int32_t nb, int32_t s, int32_t n_h, size_t *bytes) {
  if (!bytes || nb < 0 || s < 0 || n_h < 0 || s > (1 << 20))
    return call_fail(OASES_E_ARG, "oases_attention_bwd_workspace_bytes: bad argument");
  *bytes = attention_bwd_scratch_bytes(nb, s, n_h);
  return OASES_OK;
}

int oases_attention_bwd(int32_t nb, int32_t s, int32_t n_h, int32_t d, int32_t causal, const void *qkv,
                        const void *o, const void *dout, const float *lse, void *dqkv, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return attention_bwd_call(nb, s, n_h, d, causal, qkv, o, dout, lse, dqkv, workspace, workspace_bytes,
                            static_cast<hipStream_t>(stream));
}

const char *oases_last_call_error(void) { return g_call_err.c_str(); }

}  // extern "C"
