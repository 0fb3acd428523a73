"""Float64 definitions of one TMP shard's blocks (test infrastructure only).

A block is the Megatron-style pair "column-parallel GEMM -> (GeLU | causal
attention) -> row-parallel GEMM" followed by an AllReduce point.  In the Oases
paper (arXiv 2305.16121, Section IV) the forward operator sequence is
(F_i, C_i(F), F_j): F_i is this shard's compute up to its partial output, C_i
the AllReduce, F_j the next block.  The shard computes a partial sum P; the
AllReduce point returns Y = sum over the w ranks' partials (Section IV,
the definition of y as the sum of the x_i), so dL/dP = dL/dY (Eq. (1)).

All arrays are float64.  Activations are [T, features] with token row
r = b*s + t.  Weights use the nn.Linear layout [out, in].
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ----------------------------------------------------------------------------
# GeLU, exact (erf) form: gelu(u) = u * Phi(u)
# ----------------------------------------------------------------------------

def gelu(u):
    return 0.5 * u * (1.0 + erf(u / _SQRT2))


def gelu_grad(u):
    """d gelu / du = Phi(u) + u * phi(u)."""
    return 0.5 * (1.0 + erf(u / _SQRT2)) + u * np.exp(-0.5 * u * u) * _INV_SQRT_2PI


# GeLU, tanh form: gelu_t(u) = u/2 (1 + tanh(c (u + 0.044715 u^3))), c = sqrt(2/pi)
_C_TANH = math.sqrt(2.0 / math.pi)


def gelu_tanh(u):
    return 0.5 * u * (1.0 + np.tanh(_C_TANH * (u + 0.044715 * u ** 3)))


def gelu_tanh_grad(u):
    t = np.tanh(_C_TANH * (u + 0.044715 * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * _C_TANH * (1.0 + 3 * 0.044715 * u * u)


# ----------------------------------------------------------------------------
# replicated block tail (full transformer block): LayerNorm before the column
# GEMM, dropout + residual after the AllReduce point
# ----------------------------------------------------------------------------

def layer_norm(x, w, b, eps):
    """Row-wise (x - mean) / sqrt(var + eps) * w + b, var the biased variance."""
    mu = x.mean(axis=1, keepdims=True)
    xc = x - mu
    rstd = 1.0 / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + eps)
    return xc * rstd * w + b


def layer_norm_backward(x, w, eps, dz):
    """(dL/dx, dL/dw, dL/db) of z = layer_norm(x, w, b, eps) given dz."""
    h = x.shape[1]
    mu = x.mean(axis=1, keepdims=True)
    xc = x - mu
    rstd = 1.0 / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + eps)
    xh = xc * rstd
    gy = dz * w
    dx = rstd * (gy - gy.sum(axis=1, keepdims=True) / h - xh * (gy * xh).sum(axis=1, keepdims=True) / h)
    return dx, (dz * xh).sum(axis=0), dz.sum(axis=0)


# Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC'11): 10 rounds of two 64x64->128 multiplies on a
# 4-word counter under a 2-word key bumped by the Weyl constants each round.
_PH_M0, _PH_M1 = np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157)
_PH_W0, _PH_W1 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo64(a, b):
    """(high, low) 64-bit words of a * b for uint64 arrays (32-bit limbs)."""
    a_lo, a_hi = a & _LO32, a >> _S32
    b_lo, b_hi = b & _LO32, b >> _S32
    ll, lh, hl, hh = a_lo * b_lo, a_lo * b_hi, a_hi * b_lo, a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO32) + (hl & _LO32)
    return hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32), a * b


def philox4x64(c0, c1, c2, c3, k0, k1):
    """Philox4x64-10 of counters (c0, c1, c2, c3) (uint64 arrays or scalars)
    under key (k0, k1); returns the 4 output words."""
    c = [np.asarray(v, dtype=np.uint64) for v in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(k0), np.uint64(k1)
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo64(_PH_M0, c[0])
            hi1, lo1 = _mulhilo64(_PH_M1, c[2])
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
            k0, k1 = k0 + _PH_W0, k1 + _PH_W1
    return c


def dropout_keep(rows, h, layer, sb, seed, drop_q):
    """Keep mask [rows, h] of the dropout after block `layer`'s AllReduce
    point for sub-batch sb.  Element e = row*h + col takes output word e % 4
    of Philox4x64-10 at counter (e // 4, sb, 0, 0) under key (seed, layer)
    and is kept iff that word < (65536 - drop_q) * 2^48 (drop probability
    drop_q / 65536, decided in integers)."""
    if drop_q == 0:
        return np.ones((rows, h), dtype=bool)
    n = rows * h
    n4 = (n + 3) // 4
    words = philox4x64(np.arange(n4, dtype=np.uint64), sb, 0, 0, seed, layer)
    thr = np.uint64((65536 - drop_q) << 48)
    keep = np.stack([wd < thr for wd in words], axis=1).reshape(-1)[:n]
    return keep.reshape(rows, h)


def dropout_residual(x, s, keep, drop_q):
    """x + dropout(s): kept elements of s scaled by 1 / (1 - p)."""
    return x + np.where(keep, s * (65536.0 / (65536 - drop_q)), 0.0)


# ----------------------------------------------------------------------------
# causal multi-head attention on [nb, nh, s, d] tensors
# ----------------------------------------------------------------------------

def attention_fwd(q, k, v, causal=True):
    """O = softmax(Q K^T / sqrt(d) + mask) V.  Key j is visible to query i iff
    j <= i when causal.  Returns (O, P) with P the softmax matrix."""
    d = q.shape[-1]
    s = q.shape[-2]
    scores = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d)
    if causal:
        mask = np.triu(np.ones((s, s), dtype=bool), k=1)
        scores = np.where(mask, -np.inf, scores)
    scores = scores - scores.max(axis=-1, keepdims=True)
    e = np.exp(scores)
    p = e / e.sum(axis=-1, keepdims=True)
    return np.matmul(p, v), p


def attention_bwd(q, k, v, p, do):
    """Gradients of O = P V with P = softmax(Q K^T / sqrt(d) + mask).

    dV = P^T dO;  dP = dO V^T;  dS = P * (dP - rowsum(P * dP));
    dQ = dS K / sqrt(d);  dK = dS^T Q / sqrt(d).
    """
    d = q.shape[-1]
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) / math.sqrt(d)
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) / math.sqrt(d)
    return dq, dk, dv


def split_heads(m, nb, s, nh, d):
    """[nb*s, nh*d] (head-major columns) -> [nb, nh, s, d]."""
    return m.reshape(nb, s, nh, d).transpose(0, 2, 1, 3)


def merge_heads(t):
    """[nb, nh, s, d] -> [nb*s, nh*d]."""
    nb, nh, s, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(nb * s, nh * d)


# ----------------------------------------------------------------------------
# shard blocks.  forward returns (P, acts); backward takes dP = dY (Eq. (1))
# ----------------------------------------------------------------------------

def ffn_forward(x, w_in, b_in, w_out, tanh_gelu=False):
    """Column-parallel GEMM + bias + GeLU, then the row-parallel GEMM."""
    u = x @ w_in.T + b_in
    hdn = gelu_tanh(u) if tanh_gelu else gelu(u)
    return hdn @ w_out.T, {"U": u, "H": hdn}


def ffn_backward(x, acts, dp, w_in, w_out, tanh_gelu=False):
    dh = dp @ w_out
    du = dh * (gelu_tanh_grad(acts["U"]) if tanh_gelu else gelu_grad(acts["U"]))
    return du @ w_in, {"dw_in": du.T @ x, "db_in": du.sum(axis=0), "dw_out": dp.T @ acts["H"]}


def attn_forward(x, w_qkv, b_qkv, w_o, nb, s, nh, d, causal=True):
    """QKV column-parallel GEMM + bias ([Q | K | V], head-major), causal
    attention per (sequence, head), then the out-projection row-parallel GEMM."""
    a = nh * d
    qkv = x @ w_qkv.T + b_qkv
    q = split_heads(qkv[:, :a], nb, s, nh, d)
    k = split_heads(qkv[:, a:2 * a], nb, s, nh, d)
    v = split_heads(qkv[:, 2 * a:], nb, s, nh, d)
    o4, p = attention_fwd(q, k, v, causal)
    o = merge_heads(o4)
    return o @ w_o.T, {"QKV": qkv, "O": o, "Pm": p, "q": q, "k": k, "v": v}


def attn_backward(x, acts, dp, w_qkv, w_o, nb, s, nh, d):
    do = dp @ w_o
    dw_o = dp.T @ acts["O"]
    dq, dk, dv = attention_bwd(acts["q"], acts["k"], acts["v"], acts["Pm"],
                               split_heads(do, nb, s, nh, d))
    dqkv = np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv)], axis=1)
    return dqkv @ w_qkv, {"dw_in": dqkv.T @ x, "db_in": dqkv.sum(axis=0), "dw_out": dw_o}


def allreduce_point(own, peers):
    """y = sum of the w inputs (own partial first, then the w-1 peers)."""
    y = own.copy()
    for pk in peers:
        y = y + pk
    return y


# ----------------------------------------------------------------------------
# dispatch by block kind (0 = attention, 1 = FFN)
# ----------------------------------------------------------------------------

def block_forward(kind, x, w_in, b_in, w_out, nb, s, nh, d, causal=True, tanh_gelu=False):
    if kind == 0:
        return attn_forward(x, w_in, b_in, w_out, nb, s, nh, d, causal)
    return ffn_forward(x, w_in, b_in, w_out, tanh_gelu)


def block_backward(kind, x, acts, dp, w_in, w_out, nb, s, nh, d, tanh_gelu=False):
    if kind == 0:
        return attn_backward(x, acts, dp, w_in, w_out, nb, s, nh, d)
    return ffn_backward(x, acts, dp, w_in, w_out, tanh_gelu)
