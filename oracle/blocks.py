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

def ffn_forward(x, w_in, b_in, w_out):
    """Column-parallel GEMM + bias + GeLU, then the row-parallel GEMM."""
    u = x @ w_in.T + b_in
    hdn = gelu(u)
    return hdn @ w_out.T, {"U": u, "H": hdn}


def ffn_backward(x, acts, dp, w_in, w_out):
    dh = dp @ w_out
    du = dh * gelu_grad(acts["U"])
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

def block_forward(kind, x, w_in, b_in, w_out, nb, s, nh, d, causal=True):
    if kind == 0:
        return attn_forward(x, w_in, b_in, w_out, nb, s, nh, d, causal)
    return ffn_forward(x, w_in, b_in, w_out)


def block_backward(kind, x, acts, dp, w_in, w_out, nb, s, nh, d):
    if kind == 0:
        return attn_backward(x, acts, dp, w_in, w_out, nb, s, nh, d)
    return ffn_backward(x, acts, dp, w_in, w_out)
