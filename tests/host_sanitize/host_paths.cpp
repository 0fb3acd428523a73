// Host paths of liboases_shard's executor that need no GPU: configuration,
// workspace and buffer validation, op lists, call-order checks and the
// context-free entry points' argument checks.  Built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host side and run on the CPU; any
// report, or a check below that fails, ends the program with a nonzero
// status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "oases_shard.h"

static int g_fail = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

static oases_config pair_config(const int32_t *blocks, int L) {
  oases_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = L;
  c.blocks = blocks;
  c.micro_batch = 8;
  c.seq = 512;
  c.hidden = 1024;
  c.heads_per_shard = 4;
  c.head_dim = 64;
  c.ffn_shard = 1024;
  c.tmp_width = 4;
  c.dtype = OASES_BF16;
  c.causal = 1;
  c.ln_eps = 1e-5f;
  return c;
}

// an aligned fake device address: bind checks pointers, it never reads them
static void *fake(uintptr_t i) { return reinterpret_cast<void *>((uintptr_t)0x100000 * (i + 1)); }

int main() {
  const int32_t pair[2] = {OASES_ATTN, OASES_FFN};
  int32_t stack[8];
  for (int l = 0; l < 8; ++l) stack[l] = l % 2 ? OASES_FFN : OASES_ATTN;

  // ---- configuration checks ----
  oases_ctx *ctx = nullptr;
  EXPECT(oases_create(nullptr, &ctx) == OASES_E_ARG);
  EXPECT(std::strlen(oases_last_call_error()) > 0);
  oases_config c = pair_config(pair, 2);
  EXPECT(oases_create(&c, nullptr) == OASES_E_ARG);
  {
    oases_config b = c; b.micro_batch = 7;
    EXPECT(oases_create(&b, &ctx) == OASES_E_SHAPE && ctx == nullptr);
    b = c; b.head_dim = 96;
    EXPECT(oases_create(&b, &ctx) == OASES_E_SHAPE);
    b = c; b.n_layers = 0;
    EXPECT(oases_create(&b, &ctx) == OASES_E_SHAPE);
    b = c; b.n_layers = 65;
    EXPECT(oases_create(&b, &ctx) == OASES_E_SHAPE);
    b = c; b.hidden = 1000;
    EXPECT(oases_create(&b, &ctx) == OASES_E_SHAPE);
    b = c; b.dtype = OASES_F32;
    EXPECT(oases_create(&b, &ctx) == OASES_E_UNSUPPORTED);
  }

  // ---- workspace sizes: every mode, bare and full blocks ----
  for (int full = 0; full < 2; ++full) {
    oases_config b = pair_config(stack, 8);
    b.full_block = full;
    b.drop_q = full ? 6554 : 0;
    size_t prev = 0;
    for (int m = 0; m <= 5; ++m) {
      size_t bytes = 0;
      EXPECT(oases_workspace_bytes(&b, m, &bytes) == OASES_OK && bytes > 0);
      if (m == OASES_SERIAL_NO_RECOMPUTE) {
        size_t fine = 0;
        oases_workspace_bytes(&b, OASES_SERIAL_FINE, &fine);
        EXPECT(bytes > fine);
      }
      prev = bytes;
    }
    (void)prev;
    size_t bytes = 0;
    EXPECT(oases_workspace_bytes(&b, 6, &bytes) == OASES_E_ARG);
    EXPECT(oases_workspace_bytes(&b, 0, nullptr) == OASES_E_ARG);
  }

  // ---- a context: binding, op lists, call order ----
  EXPECT(oases_create(&c, &ctx) == OASES_OK && ctx != nullptr);
  size_t ws = 0;
  EXPECT(oases_workspace_bytes(&c, OASES_SERIAL_FINE, &ws) == OASES_OK);
  oases_buffers buf;
  std::memset(&buf, 0, sizeof buf);
  buf.x = fake(0); buf.y = fake(1); buf.dy = fake(2); buf.dx = fake(3); buf.ckpt = fake(4);
  buf.peers_fwd = fake(5); buf.peers_bwd = fake(6); buf.workspace = fake(7); buf.workspace_bytes = ws;
  std::vector<oases_layer_params> prm(2);
  for (int l = 0; l < 2; ++l) {
    std::memset(&prm[l], 0, sizeof prm[l]);
    prm[l].w_in = fake(10 + 6 * l); prm[l].b_in = fake(11 + 6 * l); prm[l].w_out = fake(12 + 6 * l);
    prm[l].dw_in = fake(13 + 6 * l); prm[l].db_in = fake(14 + 6 * l); prm[l].dw_out = fake(15 + 6 * l);
  }
  EXPECT(layer_fwd(ctx, 0, 0) == OASES_E_STATE);  // not bound
  EXPECT(oases_bind(ctx, nullptr, prm.data()) == OASES_E_ARG);
  {
    oases_buffers b = buf; b.dy = reinterpret_cast<void *>((uintptr_t)0x100008);
    EXPECT(oases_bind(ctx, &b, prm.data()) == OASES_E_ALIGN);
    b = buf; b.workspace_bytes = ws - 1;
    EXPECT(oases_bind(ctx, &b, prm.data()) == OASES_E_ARG);
    b = buf; b.peers_bwd = nullptr;
    EXPECT(oases_bind(ctx, &b, prm.data()) == OASES_E_ARG);
    std::vector<oases_layer_params> p2 = prm;
    p2[1].dw_out = nullptr;
    EXPECT(oases_bind(ctx, &buf, p2.data()) == OASES_E_ARG);
    EXPECT(std::strstr(oases_last_error(ctx), "dw_out") != nullptr);
  }
  EXPECT(oases_bind(ctx, &buf, prm.data()) == OASES_OK);
  EXPECT(layer_fwd(ctx, 0, 0) == OASES_E_STATE);  // streams not set
  EXPECT(layer_fwd(ctx, 2, 0) == OASES_E_ARG);
  EXPECT(layer_fwd(ctx, 0, 2) == OASES_E_ARG);
  EXPECT(layer_bwd_recompute(ctx, 1, 0) == OASES_E_STATE);  // before the forward
  EXPECT(schedule_step(ctx, OASES_OVERLAP_FINE, 0) == OASES_E_STATE);
  EXPECT(schedule_step(ctx, 9, 0) == OASES_E_ARG);
  for (int m = 0; m <= 5; ++m) {
    int32_t n = 0;
    EXPECT(oases_schedule_ops(ctx, m, nullptr, 0, &n) == OASES_OK && n > 0);
    std::vector<int32_t> ops(4 * (size_t)n);
    int32_t n2 = 0;
    EXPECT(oases_schedule_ops(ctx, m, ops.data(), n, &n2) == OASES_OK && n2 == n);
    int comm = 0;
    for (int i = 0; i < n; ++i) {
      const int k = ops[4 * i];
      EXPECT(k >= 0 && k <= 6);
      EXPECT(ops[4 * i + 1] >= 0 && ops[4 * i + 1] < 2 && (ops[4 * i + 2] == 0 || ops[4 * i + 2] == 1));
      comm += k == 1 || k == 3 || k == 5;
    }
    // per layer and sub-batch: C(F), C(B), and C(R) only in the default-recompute mode
    EXPECT(comm == 2 * 2 * (m == OASES_SERIAL_DEFAULT_RECOMPUTE ? 3 : 2));
    // a buffer shorter than the list: only cap ops are written
    std::vector<int32_t> small(4, -7);
    EXPECT(oases_schedule_ops(ctx, m, small.data(), 1, &n2) == OASES_OK && n2 == n);
  }
  oases_destroy(ctx);
  oases_destroy(nullptr);

  // ---- sub-batch streams cool-down: from 64 MiB of AllReduce-point inputs
  // up, sub-batch 1's B_dW of layer 0 is listed on the compute stream (0) ----
  for (int big = 0; big < 2; ++big) {
    oases_config b = pair_config(pair, 2);
    if (big) {  // the 8192-hidden pair shard: 2048 x 8192 x 8 bf16 = 256 MiB per point
      b.micro_batch = 2; b.seq = 2048; b.hidden = 8192; b.heads_per_shard = 8; b.head_dim = 128;
      b.ffn_shard = 4096; b.tmp_width = 8;
    }
    oases_ctx *cx = nullptr;
    EXPECT(oases_create(&b, &cx) == OASES_OK);
    if (!cx) continue;
    int32_t n = 0;
    EXPECT(oases_schedule_ops(cx, OASES_OVERLAP_STREAMS, nullptr, 0, &n) == OASES_OK);
    std::vector<int32_t> ops(4 * (size_t)n);
    EXPECT(oases_schedule_ops(cx, OASES_OVERLAP_STREAMS, ops.data(), n, &n) == OASES_OK);
    for (int i = 0; i < n; ++i) {
      const int k = ops[4 * i], l = ops[4 * i + 1], sb = ops[4 * i + 2], st = ops[4 * i + 3];
      EXPECT(st == ((big && k == 6 && l == 0) ? 0 : sb));
    }
    oases_destroy(cx);
  }

  // ---- context-free entry points: argument checks (no launch) ----
  size_t need = 0;
  EXPECT(oases_attention_bwd_workspace_bytes(2, 100, 3, &need) == OASES_OK && need > 0);
  EXPECT(oases_attention_bwd_workspace_bytes(-1, 100, 3, &need) == OASES_E_ARG);
  EXPECT(oases_attention_bwd(1, 8, 1, 96, 1, fake(0), fake(1), fake(2), (const float *)fake(3), fake(4),
                             fake(5), 1 << 20, nullptr) == OASES_E_ARG);
  EXPECT(oases_attention_bwd(1, 8, 1, 64, 1, fake(0), fake(1), nullptr, (const float *)fake(3), fake(4),
                             fake(5), 1 << 20, nullptr) == OASES_E_ARG);
  EXPECT(oases_attention_bwd(1, 8, 1, 64, 1, fake(0), fake(1), fake(2), (const float *)fake(3), fake(4),
                             fake(5), 16, nullptr) == OASES_E_ARG);
  EXPECT(std::strstr(oases_last_call_error(), "need") != nullptr);
  EXPECT(oases_attention_bwd(0, 8, 1, 64, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                             nullptr) == OASES_OK);  // empty
  EXPECT(oases_gemm(OASES_BF16, 1, 0, 4, 8, 8, 8, fake(0), 8, fake(1), 8, fake(2), 8, nullptr, nullptr,
                    nullptr, 0, 0, nullptr) == OASES_E_UNSUPPORTED);
  EXPECT(oases_gemm(OASES_BF16, 0, 0, 0, 8, 12, 8, fake(0), 8, fake(1), 8, fake(2), 16, nullptr, nullptr,
                    nullptr, 0, 0, nullptr) == OASES_E_ARG);
  EXPECT(oases_allreduce_point(OASES_BF16, fake(0), fake(1), 8, 1, fake(2), 12, nullptr) == OASES_E_ARG);
  EXPECT(oases_mfma_probe(0, 1, nullptr, nullptr) == OASES_E_ARG);
  EXPECT(oases_gemm_tile_variant(23) == OASES_E_ARG);
  EXPECT(oases_attention_variant(10) == OASES_E_ARG);
  EXPECT(oases_sum_grid_cap(0) == OASES_E_ARG);
  EXPECT(oases_sum_variant(3) == OASES_E_ARG);
  EXPECT(oases_sum_variant(-1) == OASES_E_ARG);

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host paths OK\n");
  return 0;
}
