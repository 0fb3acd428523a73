"""Seeded synthetic inputs for one tensor-model-parallel (TMP) shard of a
transformer layer stack.

This module is shared by the CPU oracle and by the GPU path, and it holds none
of the method's arithmetic: it only draws numbers, rounds them to the storage
type of a configuration and describes shapes.  Every tensor is drawn from
``numpy.random.default_rng([seed, kind, layer, sub_batch, k])`` in float64,
scaled by its standard deviation, rounded to float32 (round-to-nearest-even)
and, for bf16 configurations, rounded once more from float32 to bf16
(round-to-nearest-even on the float32 bit pattern).  Both sides consume the
rounded values, so they see identical inputs.

Shapes follow the nn.Linear convention ``[out_features, in_features]``:

* ``x``            [B*s, h]    layer-0 input, token row r = b*s + t
* ``g``            [B*s, h]    upstream gradient dL/dY of the top layer
* layer l weights  ``w_in``  [N_in, h]   (N_in = 3a for attention, f_s for FFN)
                   ``b_in``  [N_in]
                   ``w_out`` [h, N_mid]  (N_mid = a for attention, f_s for FFN)
* peer partials    [L, 2, w-1, T_sb, h] for the forward and for the backward
  AllReduce points, standing in for the other w-1 ranks' contributions.

Sub-batch k is rows [k*T_sb, (k+1)*T_sb) of a [B*s, h] tensor (the batch is
split along its batch dimension), with T_sb = (B/2)*s.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ATTN = 0
FFN = 1
F32 = 0
BF16 = 1

# tensor kinds (part of the seed tuple)
K_X, K_G, K_W_IN, K_B_IN, K_W_OUT, K_PEER_F, K_PEER_B = 1, 2, 10, 11, 12, 20, 21
K_LN_W, K_LN_B = 13, 14


@dataclasses.dataclass(frozen=True)
class ShardConfig:
    """One TMP shard of a stack of attention / FFN blocks.

    blocks         per-layer block kind (ATTN or FFN), bottom to top
    micro_batch    B, even (split into two sub-batches of B/2 sequences)
    seq            s
    hidden         h
    heads_per_shard n_s, head_dim d (a = n_s*d)
    ffn_shard      f_s, FFN columns held by this shard
    tmp_width      w, number of TMP ranks summed at an AllReduce point
    dtype          F32 or BF16 (storage type of every activation and weight)
    full_block     wrap every block in the replicated tail of a transformer
                   layer: LayerNorm (weights ln_w, ln_b) before the column
                   GEMM, dropout (drop probability drop_q / 65536, keyed by
                   drop_seed) and the residual add after the AllReduce point
    gelu_tanh      FFN GeLU in its tanh form instead of the exact (erf) form
    """
    name: str
    blocks: tuple
    micro_batch: int
    seq: int
    hidden: int
    heads_per_shard: int
    head_dim: int
    ffn_shard: int
    tmp_width: int
    dtype: int
    causal: bool = True
    w_std: float = 0.02
    bias_std: float = 0.0
    seed: int = 20250625
    full_block: bool = False
    drop_q: int = 0
    drop_seed: int = 77
    ln_eps: float = 1e-5
    ln_std: float = 0.1
    gelu_tanh: bool = False

    @property
    def n_layers(self) -> int:
        return len(self.blocks)

    @property
    def tokens(self) -> int:
        return self.micro_batch * self.seq

    @property
    def t_sb(self) -> int:
        return (self.micro_batch // 2) * self.seq

    @property
    def attn_width(self) -> int:
        return self.heads_per_shard * self.head_dim

    def n_in(self, layer: int) -> int:
        return 3 * self.attn_width if self.blocks[layer] == ATTN else self.ffn_shard

    def n_mid(self, layer: int) -> int:
        return self.attn_width if self.blocks[layer] == ATTN else self.ffn_shard

    def with_(self, **kw) -> "ShardConfig":
        return dataclasses.replace(self, **kw)


def _preset(idx, name, **kw):
    return ShardConfig(name=name, seed=20250625 + idx, **kw)


# The five workloads: a small fp32 FFN block and four bf16 layer stacks.
PRESETS = {
    "c1_ffn_fp32": _preset(0, "c1_ffn_fp32", blocks=(FFN,), micro_batch=2, seq=32, hidden=64,
                           heads_per_shard=1, head_dim=64, ffn_shard=128, tmp_width=2, dtype=F32),
    "c2_pair_h1024": _preset(1, "c2_pair_h1024", blocks=(ATTN, FFN), micro_batch=8, seq=512,
                             hidden=1024, heads_per_shard=4, head_dim=64, ffn_shard=1024,
                             tmp_width=4, dtype=BF16),
    "c3_pair_h4096": _preset(2, "c3_pair_h4096", blocks=(ATTN, FFN), micro_batch=4, seq=1024,
                             hidden=4096, heads_per_shard=4, head_dim=128, ffn_shard=2048,
                             tmp_width=8, dtype=BF16),
    "c4_stack8_h2048": _preset(3, "c4_stack8_h2048", blocks=(ATTN, FFN) * 4, micro_batch=8,
                               seq=1024, hidden=2048, heads_per_shard=4, head_dim=128,
                               ffn_shard=2048, tmp_width=4, dtype=BF16),
    "c5_pair_h8192": _preset(4, "c5_pair_h8192", blocks=(ATTN, FFN), micro_batch=2, seq=2048,
                             hidden=8192, heads_per_shard=8, head_dim=128, ffn_shard=4096,
                             tmp_width=8, dtype=BF16, w_std=0.01),
}
PRESET_ORDER = list(PRESETS)

# The same shapes wrapped as full transformer blocks (LayerNorm before every
# block, dropout p = 0.1 and the residual add after every AllReduce point).
FULL_PRESETS = {
    "c2_full_h1024": PRESETS["c2_pair_h1024"].with_(name="c2_full_h1024", full_block=True, drop_q=6554),
    "c5_full_h8192": PRESETS["c5_pair_h8192"].with_(name="c5_full_h8192", full_block=True, drop_q=6554),
}


# ----------------------------------------------------------------------------
# storage-type rounding of drawn values (input formatting only)
# ----------------------------------------------------------------------------

def _f32_to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def storage_to_f64(arr: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_bits_to_f64(arr) if dtype == BF16 else arr.astype(np.float64)


def draw(cfg: ShardConfig, kind: int, shape, std: float, layer: int = 0, sb: int = 0,
         k: int = 0, mean: float = 0.0) -> np.ndarray:
    """One tensor in storage form: float32 array, or uint16 bf16 bit patterns."""
    n = int(np.prod(shape))
    if std == 0.0:
        v32 = np.full(n, mean, np.float32)
    else:
        rng = np.random.default_rng([cfg.seed, kind, layer, sb, k])
        v32 = (rng.standard_normal(n) * std + mean).astype(np.float32)
    out = _f32_to_bf16_bits(v32) if cfg.dtype == BF16 else v32
    return out.reshape(shape)


@dataclasses.dataclass
class ShardInputs:
    """All inputs of one step, in storage form (see ``draw``)."""
    cfg: ShardConfig
    x: np.ndarray
    g: np.ndarray
    w_in: list
    b_in: list
    w_out: list
    peers_fwd: np.ndarray   # [L, 2, w-1, T_sb, h]
    peers_bwd: np.ndarray
    ln_w: list = None       # per layer [h] (full blocks only)
    ln_b: list = None

    def f64(self, name: str, layer: int | None = None) -> np.ndarray:
        v = getattr(self, name)
        if layer is not None:
            v = v[layer]
        return storage_to_f64(v, self.cfg.dtype)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def make_inputs(cfg: ShardConfig, zero_peers: bool = False) -> ShardInputs:
    """Draw every input of one step.  ``zero_peers`` replaces the peer partials
    by zeros (so a shard's own partial outputs are visible in Y and dX)."""
    L, h, w, T = cfg.n_layers, cfg.hidden, cfg.tmp_width, cfg.t_sb
    store = np.uint16 if cfg.dtype == BF16 else np.float32
    peers = {K_PEER_F: np.zeros((L, 2, w - 1, T, h), store),
             K_PEER_B: np.zeros((L, 2, w - 1, T, h), store)}
    jobs = []
    if not zero_peers:
        for kind in (K_PEER_F, K_PEER_B):
            for l in range(L):
                for sb in range(2):
                    for k in range(w - 1):
                        jobs.append((kind, l, sb, k))

    def fill(job):
        kind, l, sb, k = job
        peers[kind][l, sb, k] = draw(cfg, kind, (T, h), 1.0, l, sb, k)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, jobs))
        fx = ex.submit(draw, cfg, K_X, (cfg.tokens, h), 1.0)
        fg = ex.submit(draw, cfg, K_G, (cfg.tokens, h), 1.0)
        w_in, b_in, w_out = [], [], []
        for l in range(L):
            w_in.append(ex.submit(draw, cfg, K_W_IN, (cfg.n_in(l), h), cfg.w_std, l))
            b_in.append(ex.submit(draw, cfg, K_B_IN, (cfg.n_in(l),), cfg.bias_std, l))
            w_out.append(ex.submit(draw, cfg, K_W_OUT, (h, cfg.n_mid(l)), cfg.w_std, l))
        ln_w = ln_b = None
        if cfg.full_block:  # LayerNorm weight 1 + N(0, ln_std^2), bias N(0, ln_std^2)
            ln_w = [ex.submit(draw, cfg, K_LN_W, (h,), cfg.ln_std, l, 0, 0, 1.0) for l in range(L)]
            ln_b = [ex.submit(draw, cfg, K_LN_B, (h,), cfg.ln_std, l) for l in range(L)]
            ln_w, ln_b = [f.result() for f in ln_w], [f.result() for f in ln_b]
        return ShardInputs(cfg=cfg, x=fx.result(), g=fg.result(),
                           w_in=[f.result() for f in w_in], b_in=[f.result() for f in b_in],
                           w_out=[f.result() for f in w_out],
                           peers_fwd=peers[K_PEER_F], peers_bwd=peers[K_PEER_B], ln_w=ln_w, ln_b=ln_b)
