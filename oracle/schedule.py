"""Schedules of one training step and a step simulator (test infrastructure only).

Source: Oases (arXiv 2305.16121), Section IV:
  * default recompute backward (R_i, C_i(R), R_j), (B_j, B_i, C_i(B)), Fig. 4a;
  * batch split into two sub-batches whose operators pipeline, so C^0 of one
    sub-batch overlaps compute of the other, Fig. 4b;
  * fine-grained recomputation: since the gradient of each AllReduce input
    equals the gradient of its output (Eq. (1)), recomputation starts after
    the forward communication operator and C_i(R) is dropped; the backward of
    (F_i, C_i(F), F_j) becomes (R_j, B_j, R_i, B_i, C_i(B)), Fig. 4d;
  * across layers only the start positions of recompute sequences move, so no
    extra inputs are stored;
  * the executor's computation operators have Forward / Recompute / Backward,
    communication operators StartAsync / Sync; only the input of the first
    operator of each recompute sequence is stored (Algorithm 1).

Reading used here: a block l is "F_l = column GEMM -> GeLU | attention -> row
GEMM, C_l = AllReduce of the row GEMM's partial".  The replicated tail F_j is
empty (no LayerNorm / residual on this path), so block l+1 plays F_j.  With
``full_block`` configurations F_j is the tail of a transformer layer, the
same on every rank: dropout and the residual add right after the AllReduce
point, then the next block's LayerNorm before its column GEMM.  C_l(F) then
yields r_{l+1} = r_l + dropout(sum), and the backward runs the LayerNorm
backward and the residual add right after C_l(B).  The
backward of block l is split into B_dX (the data-gradient path that feeds
C_l(B)) and B_dW (weight gradients), and C_l(B) is started before B_dW.

An op is (kind, layer, sub_batch, stream) with stream 0 = compute and
1 = communication.  Kinds: F, C_F, R, C_R, B_dX, C_B, B_dW.
"""
from __future__ import annotations

import numpy as np

from gen import storage_to_f64  # input decoding only (shared seeded-input module)

from . import blocks

MODES = ("overlap_fine", "serial_fine", "serial_default", "serial_norecompute")
COMM_KINDS = ("C_F", "C_R", "C_B")


def build_ops(n_layers: int, mode: str):
    """Op list of one step, in issue order."""
    if mode not in MODES:
        raise ValueError(mode)
    side = 1 if mode == "overlap_fine" else 0
    ops = []
    for l in range(n_layers):
        for sb in (0, 1):
            ops.append(("F", l, sb, 0))
            ops.append(("C_F", l, sb, side))
    for l in reversed(range(n_layers)):
        for sb in (0, 1):
            if mode != "serial_norecompute":
                ops.append(("R", l, sb, 0))
            if mode == "serial_default":
                ops.append(("C_R", l, sb, 0))
            ops.append(("B_dX", l, sb, 0))
            ops.append(("C_B", l, sb, side))
            ops.append(("B_dW", l, sb, 0))
    return ops


def comm_ops_per_layer_sb(ops):
    """Number of communication operators per (layer, sub-batch)."""
    out = {}
    for kind, l, sb, _ in ops:
        if kind in COMM_KINDS:
            out[(l, sb)] = out.get((l, sb), 0) + 1
    return out


class _Memory(dict):
    """Tensor store that refuses reads of absent tensors."""

    def get_(self, key):
        if key not in self:
            raise KeyError(f"op reads absent tensor {key}")
        return self[key]


def run_step(inp, mode: str, keep_trace: bool = False, keep_dy: bool = False, work_dtype=np.float64):
    """Simulate one step of ``mode`` over the inputs ``inp`` (gen.ShardInputs).

    Returns a dict with Y [B*s, h], dX [B*s, h] (gradient w.r.t. the stack
    input), per-layer grads dw_in / db_in / dw_out, and the set of tensors
    stored between the forward and the backward pass.  ``work_dtype``
    float32 runs the same arithmetic in float32 (timing and diagnosis only;
    the reference is float64).
    """
    cfg = inp.cfg
    L, T, nb = cfg.n_layers, cfg.t_sb, cfg.micro_batch // 2
    nh, d, s = cfg.heads_per_shard, cfg.head_dim, cfg.seq
    f = lambda name, l=None: inp.f64(name, l).astype(work_dtype, copy=False)
    x_all, g_all = f("x"), f("g")
    w_in = [f("w_in", l) for l in range(L)]
    b_in = [f("b_in", l) for l in range(L)]
    w_out = [f("w_out", l) for l in range(L)]
    full = cfg.full_block
    ln_w = [f("ln_w", l) for l in range(L)] if full else None
    ln_b = [f("ln_b", l) for l in range(L)] if full else None

    def peers(kind, l, sb):
        src = inp.peers_fwd if kind == "fwd" else inp.peers_bwd
        return [storage_to_f64(src[l, sb, k], cfg.dtype).astype(work_dtype, copy=False)
                for k in range(cfg.tmp_width - 1)]

    mem = _Memory()
    for sb in (0, 1):
        mem[("X", 0, sb)] = x_all[sb * T:(sb + 1) * T]
        mem[("dY", L - 1, sb)] = g_all[sb * T:(sb + 1) * T]
    grads = [dict() for _ in range(L)]
    dys = {}
    keep_acts = mode == "serial_norecompute"
    stored_after_fwd = None
    trace = []
    fwd_sums = {}

    def gemm_in(l, sb):
        """The column GEMM's input: the block input, or its LayerNorm."""
        x = mem.get_(("X", l, sb))
        return blocks.layer_norm(x, ln_w[l], ln_b[l], cfg.ln_eps) if full else x

    def fwd(l, sb):
        kind = cfg.blocks[l]
        return blocks.block_forward(kind, gemm_in(l, sb), w_in[l], b_in[l], w_out[l],
                                    nb, s, nh, d, cfg.causal, cfg.gelu_tanh)

    def keep(l, sb):
        return blocks.dropout_keep(T, cfg.hidden, l, sb, cfg.drop_seed, cfg.drop_q)

    for op in build_ops(L, mode):
        kind, l, sb, _ = op
        if keep_trace:
            trace.append(op)
        if kind == "F":
            p, acts = fwd(l, sb)
            mem[("P", l, sb)] = p
            if keep_acts:
                mem[("act", l, sb)] = acts
        elif kind == "C_F":
            y = blocks.allreduce_point(mem.pop(("P", l, sb)), peers("fwd", l, sb))
            if full:
                y = blocks.dropout_residual(mem.get_(("X", l, sb)), y, keep(l, sb), cfg.drop_q)
            mem[("X", l + 1, sb) if l + 1 < L else ("Y", sb)] = y
            fwd_sums[(l, sb)] = y  # kept outside the store, only to check C_R
            if l == L - 1 and sb == 1:
                stored_after_fwd = sorted(k for k in mem if k[0] not in ("dY",))
        elif kind == "R":
            p, acts = fwd(l, sb)
            mem[("act", l, sb)] = acts
            if mode == "serial_default":
                mem[("P_R", l, sb)] = p
        elif kind == "C_R":
            y = blocks.allreduce_point(mem.pop(("P_R", l, sb)), peers("fwd", l, sb))
            if full:
                y = blocks.dropout_residual(mem.get_(("X", l, sb)), y, keep(l, sb), cfg.drop_q)
            if not np.array_equal(y, fwd_sums[(l, sb)]):
                raise AssertionError("recomputed AllReduce differs from the forward one")
        elif kind == "B_dX":
            blk = cfg.blocks[l]
            dy = mem.get_(("dY", l, sb))
            # dropout backward: the AllReduce inputs' gradient (Eq. (1))
            dp = np.where(keep(l, sb), dy * (65536.0 / (65536 - cfg.drop_q)), 0.0) if full else dy
            dxo, g = blocks.block_backward(blk, gemm_in(l, sb), mem.get_(("act", l, sb)),
                                           dp, w_in[l], w_out[l], nb, s, nh, d, cfg.gelu_tanh)
            mem[("dXown", l, sb)] = dxo
            mem[("wgrad", l, sb)] = g
        elif kind == "C_B":
            dx = blocks.allreduce_point(mem.pop(("dXown", l, sb)), peers("bwd", l, sb))
            if full:  # LayerNorm backward and the residual path, after the sum
                dxl, dlw, dlb = blocks.layer_norm_backward(mem.get_(("X", l, sb)), ln_w[l], cfg.ln_eps, dx)
                dx = mem.get_(("dY", l, sb)) + dxl
                mem.get_(("wgrad", l, sb)).update({"dln_w": dlw, "dln_b": dlb})
            mem[("dY", l - 1, sb) if l > 0 else ("dX", sb)] = dx
            if keep_dy and l > 0:
                dys[(l - 1, sb)] = dx
        elif kind == "B_dW":
            g = mem.pop(("wgrad", l, sb))
            for name, val in g.items():
                # sub-batch 0 writes, sub-batch 1 accumulates (fixed order)
                grads[l][name] = val.copy() if sb == 0 else grads[l][name] + val
            del mem[("act", l, sb)]
            del mem[("dY", l, sb)]
            if l > 0:
                del mem[("X", l, sb)]
    out = {
        "Y": np.concatenate([mem[("Y", 0)], mem[("Y", 1)]]),
        "dX": np.concatenate([mem[("dX", 0)], mem[("dX", 1)]]),
        "grads": grads,
        "stored_after_fwd": stored_after_fwd,
    }
    if keep_trace:
        out["trace"] = trace
    if keep_dy:
        out["dY"] = {l: np.concatenate([dys[(l, 0)], dys[(l, 1)]]) for l in range(L - 1)}
    return out


def run_unsplit(inp):
    """Whole-batch reference with no sub-batch split and no recomputation:
    every block's forward over all B sequences, then its backward."""
    cfg = inp.cfg
    L, nb = cfg.n_layers, cfg.micro_batch
    nh, d, s = cfg.heads_per_shard, cfg.head_dim, cfg.seq

    def peers_full(src, l):
        return [np.concatenate([storage_to_f64(src[l, sb, k], cfg.dtype) for sb in (0, 1)])
                for k in range(cfg.tmp_width - 1)]

    full, T, h = cfg.full_block, cfg.t_sb, cfg.hidden
    scale = 65536.0 / (65536 - cfg.drop_q)

    def keep_full(l):  # masks are drawn per sub-batch (sub-batch counters)
        return np.concatenate([blocks.dropout_keep(T, h, l, sb, cfg.drop_seed, cfg.drop_q) for sb in (0, 1)])

    def gemm_in(l, x):
        return blocks.layer_norm(x, inp.f64("ln_w", l), inp.f64("ln_b", l), cfg.ln_eps) if full else x

    xs, acts = [inp.f64("x")], []
    for l in range(L):
        p, a = blocks.block_forward(cfg.blocks[l], gemm_in(l, xs[-1]), inp.f64("w_in", l), inp.f64("b_in", l),
                                    inp.f64("w_out", l), nb, s, nh, d, cfg.causal, cfg.gelu_tanh)
        acts.append(a)
        y = blocks.allreduce_point(p, peers_full(inp.peers_fwd, l))
        xs.append(blocks.dropout_residual(xs[-1], y, keep_full(l), cfg.drop_q) if full else y)
    dy = inp.f64("g")
    grads = [None] * L
    for l in reversed(range(L)):
        dp = np.where(keep_full(l), dy * scale, 0.0) if full else dy
        dxo, grads[l] = blocks.block_backward(cfg.blocks[l], gemm_in(l, xs[l]), acts[l], dp,
                                              inp.f64("w_in", l), inp.f64("w_out", l),
                                              nb, s, nh, d, cfg.gelu_tanh)
        dz = blocks.allreduce_point(dxo, peers_full(inp.peers_bwd, l))
        if full:
            dxl, grads[l]["dln_w"], grads[l]["dln_b"] = blocks.layer_norm_backward(
                xs[l], inp.f64("ln_w", l), cfg.ln_eps, dz)
            dy = dy + dxl
        else:
            dy = dz
    return {"Y": xs[-1], "dX": dy, "grads": grads}
