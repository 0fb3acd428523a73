"""Pins of the CPU oracle against facts that do not come from the oracle itself:
textbook values, closed forms, brute force on tiny inputs, finite differences,
and the invariants the Oases schedule section states (Eq. (1), the comm-count
reduction of fine-grained recomputation, and "no extra stored inputs")."""
import dataclasses
import math

import numpy as np
import pytest

import gen
from oracle import blocks, schedule, sums

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------
# GeLU
# ----------------------------------------------------------------------------

# Standard normal CDF values (any statistics table): Phi(1), Phi(2), Phi(-1), Phi(1.96)
PHI = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -1.0: 0.15865525393145707,
       1.96: 0.9750021048517795}


def test_gelu_table_values():
    for u, phi in PHI.items():
        assert blocks.gelu(np.array(u)) == pytest.approx(u * phi, rel=1e-14, abs=1e-15)


def test_gelu_special_values_and_symmetry():
    assert blocks.gelu(np.array(0.0)) == 0.0
    assert blocks.gelu_grad(np.array(0.0)) == 0.5
    u = RNG.standard_normal(1000) * 3
    # Phi(u) + Phi(-u) = 1  =>  gelu(u) - gelu(-u) = u
    np.testing.assert_allclose(blocks.gelu(u) - blocks.gelu(-u), u, rtol=0, atol=1e-14)
    # gelu'(u) + gelu'(-u) = 1 (the u*phi(u) terms cancel, the Phi terms sum to 1)
    np.testing.assert_allclose(blocks.gelu_grad(u) + blocks.gelu_grad(-u), 1.0, atol=1e-14)
    assert blocks.gelu(np.array(40.0)) == 40.0
    assert blocks.gelu(np.array(-40.0)) == 0.0


def test_gelu_grad_finite_difference():
    u = np.linspace(-5, 5, 101)
    eps = 1e-6
    fd = (blocks.gelu(u + eps) - blocks.gelu(u - eps)) / (2 * eps)
    np.testing.assert_allclose(blocks.gelu_grad(u), fd, rtol=1e-8, atol=1e-9)


# ----------------------------------------------------------------------------
# causal attention
# ----------------------------------------------------------------------------

def _attention_loops(q, k, v, causal):
    """Pure-Python per-query loops: scores, max shift, exp, normalise."""
    nb, nh, s, d = q.shape
    out = np.zeros_like(q)
    for b in range(nb):
        for h in range(nh):
            for i in range(s):
                visible = range(i + 1) if causal else range(s)
                sc = [sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) / math.sqrt(d)
                      for j in visible]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = sum(e)
                for c in range(d):
                    out[b, h, i, c] = sum(e[n] * v[b, h, j, c] for n, j in enumerate(visible)) / tot
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_attention_brute_force(causal):
    q, k, v = (RNG.standard_normal((1, 2, 5, 3)) for _ in range(3))
    o, p = blocks.attention_fwd(q, k, v, causal)
    np.testing.assert_allclose(o, _attention_loops(q, k, v, causal), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-15)
    if causal:
        assert np.all(np.triu(p[0, 0], 1) == 0)


def test_attention_special_cases():
    v = RNG.standard_normal((2, 3, 6, 4))
    k = RNG.standard_normal((2, 3, 6, 4))
    # s = 1: the only visible key is the query's own position
    o1, _ = blocks.attention_fwd(RNG.standard_normal((2, 3, 1, 4)), k[:, :, :1], v[:, :, :1])
    np.testing.assert_array_equal(o1, v[:, :, :1])
    # Q = 0: uniform weights over visible keys -> prefix mean of V
    o0, _ = blocks.attention_fwd(np.zeros_like(v), k, v, causal=True)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, 7)[None, None, :, None]
    np.testing.assert_allclose(o0, prefix_mean, rtol=1e-14, atol=1e-15)
    # non-causal with identical keys -> plain mean over all positions
    kk = np.repeat(k[:, :, :1], 6, axis=2)
    on, _ = blocks.attention_fwd(RNG.standard_normal(v.shape), kk, v, causal=False)
    np.testing.assert_allclose(on, np.broadcast_to(v.mean(2, keepdims=True), v.shape), atol=1e-14)


def test_attention_causality():
    q, k, v = (RNG.standard_normal((1, 1, 8, 4)) for _ in range(3))
    o, _ = blocks.attention_fwd(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5:] += 3.0
    v2[:, :, 5:] -= 2.0
    o2, _ = blocks.attention_fwd(q, k2, v2)
    np.testing.assert_array_equal(o[:, :, :5], o2[:, :, :5])
    assert not np.allclose(o[:, :, 5:], o2[:, :, 5:])


@pytest.mark.parametrize("causal", [True, False])
def test_attention_bwd_finite_difference(causal):
    q, k, v, do = (RNG.standard_normal((2, 2, 5, 3)) for _ in range(4))
    _, p = blocks.attention_fwd(q, k, v, causal)
    dq, dk, dv = blocks.attention_bwd(q, k, v, p, do)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = np.sum(blocks.attention_fwd(q, k, v, causal)[0] * do)
            arr[idx] = old - eps
            lm = np.sum(blocks.attention_fwd(q, k, v, causal)[0] * do)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


# ----------------------------------------------------------------------------
# blocks: finite differences of the shard's partial output
# ----------------------------------------------------------------------------

NB, S, H, NH, D, FS = 2, 4, 8, 2, 4, 16


def _block_params(kind):
    n_in = 3 * NH * D if kind == gen.ATTN else FS
    n_mid = NH * D if kind == gen.ATTN else FS
    return (RNG.standard_normal((NB * S, H)), 0.3 * RNG.standard_normal((n_in, H)),
            0.1 * RNG.standard_normal(n_in), 0.3 * RNG.standard_normal((H, n_mid)))


@pytest.mark.parametrize("kind", [gen.ATTN, gen.FFN])
def test_block_backward_finite_difference(kind):
    x, w_in, b_in, w_out = _block_params(kind)
    gp = RNG.standard_normal((NB * S, H))

    def loss():
        p, _ = blocks.block_forward(kind, x, w_in, b_in, w_out, NB, S, NH, D)
        return np.sum(p * gp)

    _, acts = blocks.block_forward(kind, x, w_in, b_in, w_out, NB, S, NH, D)
    dx, g = blocks.block_backward(kind, x, acts, gp, w_in, w_out, NB, S, NH, D)
    eps = 1e-6
    for arr, grad in ((x, dx), (w_in, g["dw_in"]), (b_in, g["db_in"]), (w_out, g["dw_out"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss()
            arr[idx] = old - eps
            lm = loss()
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


# ----------------------------------------------------------------------------
# whole step: finite differences, Eq. (1), schedules, sharding
# ----------------------------------------------------------------------------

def _tiny_cfg(blocks_=(gen.ATTN, gen.FFN), w=3, **kw):
    base = dict(name="tiny", blocks=blocks_, micro_batch=4, seq=3, hidden=8, heads_per_shard=2,
                head_dim=4, ffn_shard=16, tmp_width=w, dtype=gen.F32, w_std=0.3,
                bias_std=0.1, seed=99)
    base.update(kw)
    return gen.ShardConfig(**base)


def _f64_inputs(cfg, zero_bwd_peers=True):
    """Inputs held as float64 arrays so finite differences can perturb them.

    The backward peer partials stand in for the other ranks' contributions to
    dX; they are constants, not derivatives of L, so a finite-difference check
    of L = <Y_top, G> holds only with them at zero (the forward peers are
    additive constants of the forward and may stay)."""
    inp = gen.make_inputs(cfg)
    f = lambda a: a.astype(np.float64)
    pb = np.zeros_like(f(inp.peers_bwd)) if zero_bwd_peers else f(inp.peers_bwd)
    ln = {}
    if cfg.full_block:
        ln = dict(ln_w=[f(a) for a in inp.ln_w], ln_b=[f(a) for a in inp.ln_b])
    return dataclasses.replace(inp, x=f(inp.x), g=f(inp.g), w_in=[f(a) for a in inp.w_in],
                               b_in=[f(a) for a in inp.b_in], w_out=[f(a) for a in inp.w_out],
                               peers_fwd=f(inp.peers_fwd), peers_bwd=pb, **ln)


def _step_loss(inp):
    y = schedule.run_unsplit(inp)["Y"]
    return float(np.sum(y * inp.g))


def test_step_directional_finite_difference():
    """<grad, v> equals the directional derivative of L = <Y_top, G> for a
    random direction over the input and every weight of every layer."""
    cfg = _tiny_cfg()
    inp = _f64_inputs(cfg)
    params = [("x", None)] + [(n, l) for l in range(cfg.n_layers) for n in ("w_in", "b_in", "w_out")]

    def get(i, name, l):
        return getattr(i, name) if l is None else getattr(i, name)[l]

    dirs = {p: RNG.standard_normal(get(inp, *p).shape) for p in params}
    for mode in schedule.MODES:
        out = schedule.run_step(inp, mode)
        analytic = np.sum(out["dX"] * dirs[("x", None)])
        for l in range(cfg.n_layers):
            for n, gname in (("w_in", "dw_in"), ("b_in", "db_in"), ("w_out", "dw_out")):
                analytic += np.sum(out["grads"][l][gname] * dirs[(n, l)])
        eps = 1e-6
        vals = []
        for sgn in (1, -1):
            pert = _f64_inputs(cfg)
            for (n, l), dvec in dirs.items():
                get(pert, n, l)[...] += sgn * eps * dvec
            vals.append(_step_loss(pert))
        fd = (vals[0] - vals[1]) / (2 * eps)
        assert analytic == pytest.approx(fd, rel=1e-7), mode


def test_eq1_allreduce_input_gradient_equals_output_gradient():
    """The gradient of L w.r.t. any AllReduce input (own partial or a peer's)
    equals the gradient w.r.t. the AllReduce output: for the top point it is
    G; for the point below it is the dY the backward feeds to the layer above."""
    cfg = _tiny_cfg(w=3)
    inp = _f64_inputs(cfg)
    out = schedule.run_step(inp, "serial_fine", keep_dy=True)
    T, eps = cfg.t_sb, 1e-6
    for l, expect in ((1, inp.g), (0, out["dY"][0])):
        for sb in (0, 1):
            for k in range(cfg.tmp_width - 1):
                for (i, j) in ((0, 0), (T - 1, cfg.hidden - 1), (1, 3)):
                    vals = []
                    for sgn in (1, -1):
                        pert = _f64_inputs(cfg)
                        pert.peers_fwd[l, sb, k, i, j] += sgn * eps
                        vals.append(_step_loss(pert))
                    fd = (vals[0] - vals[1]) / (2 * eps)
                    assert fd == pytest.approx(expect[sb * T + i, j], rel=1e-6, abs=1e-9)


def test_schedules_identical_and_comm_counts():
    cfg = _tiny_cfg(blocks_=(gen.ATTN, gen.FFN, gen.ATTN, gen.FFN))
    inp = _f64_inputs(cfg, zero_bwd_peers=False)
    ref = schedule.run_step(inp, "serial_norecompute")
    for mode in schedule.MODES:
        out = schedule.run_step(inp, mode)
        np.testing.assert_array_equal(out["Y"], ref["Y"])
        np.testing.assert_array_equal(out["dX"], ref["dX"])
        for l in range(cfg.n_layers):
            for n in ("dw_in", "db_in", "dw_out"):
                np.testing.assert_array_equal(out["grads"][l][n], ref["grads"][l][n])
    unsplit = schedule.run_unsplit(inp)
    np.testing.assert_allclose(ref["Y"], unsplit["Y"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ref["dX"], unsplit["dX"], rtol=1e-13, atol=1e-13)
    for l in range(cfg.n_layers):
        for n in ("dw_in", "db_in", "dw_out"):
            np.testing.assert_allclose(ref["grads"][l][n], unsplit["grads"][l][n], rtol=1e-12,
                                       atol=1e-13)
    # fine-grained recompute drops C(R): three comm ops per layer and sub-batch become two
    L = cfg.n_layers
    for mode, n in (("serial_default", 3), ("serial_fine", 2), ("overlap_fine", 2)):
        counts = schedule.comm_ops_per_layer_sb(schedule.build_ops(L, mode))
        assert set(counts.values()) == {n} and len(counts) == 2 * L


def test_fine_grained_stores_no_extra_inputs():
    cfg = _tiny_cfg(blocks_=(gen.ATTN, gen.FFN, gen.ATTN))
    inp = _f64_inputs(cfg)
    stored = {m: schedule.run_step(inp, m)["stored_after_fwd"] for m in schedule.MODES}
    expect = sorted([("X", l, sb) for l in range(3) for sb in (0, 1)] + [("Y", 0), ("Y", 1)])
    for m in ("serial_default", "serial_fine", "overlap_fine"):
        assert stored[m] == expect
    assert len(stored["serial_norecompute"]) == len(expect) + 6


def test_overlap_schedule_streams():
    ops = schedule.build_ops(4, "overlap_fine")
    for kind, _, _, stream in ops:
        assert stream == (1 if kind in schedule.COMM_KINDS else 0)
    # the sub-batch-0 backward AllReduce is issued before the other sub-batch's compute
    i_cb = ops.index(("C_B", 3, 0, 1))
    assert ops.index(("R", 3, 1, 0)) > i_cb and ops.index(("B_dW", 3, 0, 0)) > i_cb
    # fine-grained backward of a block: R, B_dX, C_B, B_dW
    assert [o[0] for o in ops if o[1] == 2 and o[2] == 1 and o[0] != "F" and o[0] != "C_F"] == \
        ["R", "B_dX", "C_B", "B_dW"]


def _shard_weights(kind, full, w, k, a_or_f, hidden):
    """Slice rank k's column / row shard out of full-width weights."""
    w_in, b_in, w_out = full
    if kind == gen.FFN:
        cols = slice(k * a_or_f, (k + 1) * a_or_f)
        return w_in[cols], b_in[cols], w_out[:, cols]
    A = w * a_or_f
    rows = np.concatenate([np.arange(part * A + k * a_or_f, part * A + (k + 1) * a_or_f)
                           for part in range(3)])
    return w_in[rows], b_in[rows], w_out[:, k * a_or_f:(k + 1) * a_or_f]


@pytest.mark.parametrize("kind", [gen.ATTN, gen.FFN])
def test_sum_over_shards_equals_unsharded_block(kind):
    w, nb, s, h, nh, d, fs = 4, 2, 5, 8, 2, 4, 6
    width = nh * d if kind == gen.ATTN else fs
    n_in_full = 3 * w * width if kind == gen.ATTN else w * fs
    x = RNG.standard_normal((nb * s, h))
    full = (0.3 * RNG.standard_normal((n_in_full, h)), 0.1 * RNG.standard_normal(n_in_full),
            0.3 * RNG.standard_normal((h, w * width)))
    gp = RNG.standard_normal((nb * s, h))
    p_full, acts = blocks.block_forward(kind, x, *full, nb, s, w * nh, d)
    dx_full, g_full = blocks.block_backward(kind, x, acts, gp, full[0], full[2], nb, s, w * nh, d)
    p_sum, dx_sum = 0, 0
    for k in range(w):
        wi, bi, wo = _shard_weights(kind, full, w, k, width, h)
        pk, ak = blocks.block_forward(kind, x, wi, bi, wo, nb, s, nh, d)
        dxk, gk = blocks.block_backward(kind, x, ak, gp, wi, wo, nb, s, nh, d)
        p_sum = p_sum + pk
        dx_sum = dx_sum + dxk
        full_slices = _shard_weights(kind, (g_full["dw_in"], g_full["db_in"], g_full["dw_out"]),
                                     w, k, width, h)
        for got, want in zip((gk["dw_in"], gk["db_in"], gk["dw_out"]), full_slices):
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p_sum, p_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dx_sum, dx_full, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# storage-type sum
# ----------------------------------------------------------------------------

def _bits(v):
    return np.array([v], np.float32).view(np.uint32)[0] >> 16


def test_sum_float32_sequential_semantics():
    big = np.array([2.0 ** 24], np.float32)
    one = np.array([1.0], np.float32)
    # (2^24 + 1) rounds to 2^24 (tie to even); adding 1 again does the same
    assert sums.allreduce_point_storage(big, [one, one], False)[0] == 2.0 ** 24
    # reordering the same inputs changes the float32 result: order is part of the definition
    assert sums.allreduce_point_storage(one, [one, big], False)[0] == 2.0 ** 24 + 2


def test_sum_bf16_round_to_nearest_even():
    enc = lambda v: np.array([_bits(v)], np.uint16)
    one, zero = enc(1.0), enc(0.0)
    half_ulp = np.array([0x3B80], np.uint16)     # 2^-8 = half a bf16 ulp at 1.0
    assert sums.allreduce_point_storage(one, [half_ulp], True)[0] == 0x3F80      # tie -> even
    three_q = np.array([0x3BC0], np.uint16)      # 1.5 * 2^-8 -> above the tie
    assert sums.allreduce_point_storage(one, [three_q], True)[0] == 0x3F81
    odd = np.array([0x3F81], np.uint16)          # 1 + 2^-7 (odd mantissa) + half ulp -> up
    assert sums.allreduce_point_storage(odd, [half_ulp, zero], True)[0] == 0x3F82
    neg = np.array([0xBF80], np.uint16)          # -1 + 1 = +0
    assert sums.allreduce_point_storage(neg, [one], True)[0] == 0x0000


# ----------------------------------------------------------------------------
# full transformer block: LayerNorm, dropout (Philox4x64-10), residual, tanh GeLU
# ----------------------------------------------------------------------------

def test_philox_matches_numpy_bit_generator():
    """The oracle's Philox4x64-10 (written from the SC'11 definition) against
    numpy's Philox bit generator, which advances its 4-word counter (with
    carry) before producing each block of four words."""
    M = (1 << 64) - 1
    for key in ((0, 0), (123, 456), (M, 7)):
        for ctr in ((0, 0, 0, 0), (5, 1, 2, 3), (M - 1, 9, 0, 1)):
            bg = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(ctr, np.uint64))
            raw = bg.random_raw(8)
            c = list(ctr)
            got = []
            for _ in range(2):
                for i in range(4):  # increment with carry
                    c[i] = (c[i] + 1) & M
                    if c[i]:
                        break
                got += [int(w) for w in blocks.philox4x64(*[np.uint64(v) for v in c], *key)]
            assert got == [int(v) for v in raw], (key, ctr)


def test_dropout_mask_rate_and_layout():
    T, h = 64, 96
    assert blocks.dropout_keep(T, h, 0, 0, 5, 0).all()
    keep = blocks.dropout_keep(T, h, 1, 0, 5, 16384)  # p = 1/4
    n = keep.size
    assert abs(keep.sum() - 0.75 * n) < 5 * math.sqrt(n * 0.75 * 0.25)
    # element e = row*h + col is word e % 4 of counter e // 4 (sub-batch in word 1, layer in the key)
    for (r, c) in ((0, 0), (3, 7), (T - 1, h - 1)):
        e = r * h + c
        w = blocks.philox4x64(np.uint64(e // 4), np.uint64(0), np.uint64(0), np.uint64(0), 5, 1)[e % 4]
        assert keep[r, c] == (int(w) < (65536 - 16384) << 48)
    # sub-batches and layers draw different masks
    assert (keep != blocks.dropout_keep(T, h, 1, 1, 5, 16384)).any()
    assert (keep != blocks.dropout_keep(T, h, 2, 0, 5, 16384)).any()


def test_dropout_scale_is_inverted_dropout():
    """dropout_residual keeps an element as s / (1 - p) and drops it to 0,
    checked against scales written out by hand for p = 1/2, 1/4 and 1/8
    (2, 4/3, 8/7), and against the defining property of inverted dropout:
    averaged over many independent masks, dropout(s) has mean s."""
    T, h = 32, 64
    s = RNG.standard_normal((T, h))
    x = RNG.standard_normal((T, h))
    for drop_q, scale in ((32768, 2.0), (16384, 4.0 / 3.0), (8192, 8.0 / 7.0)):
        keep = blocks.dropout_keep(T, h, 3, 1, 77, drop_q)
        out = blocks.dropout_residual(x, s, keep, drop_q)
        assert keep.any() and (~keep).any()
        np.testing.assert_allclose(out[keep], x[keep] + s[keep] * scale, rtol=1e-15, atol=0)
        np.testing.assert_array_equal(out[~keep], x[~keep])
    # expectation over 400 masks (different layers): mean within 5 standard errors of s
    drop_q, p = 16384, 0.25
    ones = np.ones((8, 16))
    acc = np.zeros_like(ones)
    for layer in range(400):
        keep = blocks.dropout_keep(8, 16, layer, 0, 99, drop_q)
        acc += blocks.dropout_residual(np.zeros_like(ones), ones, keep, drop_q)
    mean = acc / 400
    se = math.sqrt(p / (1 - p) / 400)  # std of one draw of dropout(1) is sqrt(p / (1 - p))
    assert np.abs(mean - 1.0).max() < 5 * se


def test_layer_norm_matches_torch():
    import torch
    x, w, b = RNG.standard_normal((7, 24)) * 3 + 1, RNG.standard_normal(24), RNG.standard_normal(24)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(w),
                                         torch.from_numpy(b), 1e-5).numpy()
    np.testing.assert_allclose(blocks.layer_norm(x, w, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_backward_matches_autograd():
    import torch
    x, w, b = RNG.standard_normal((5, 16)) * 2, RNG.standard_normal(16), RNG.standard_normal(16)
    dz = RNG.standard_normal((5, 16))
    tx, tw, tb = (torch.tensor(v, requires_grad=True) for v in (x, w, b))
    torch.nn.functional.layer_norm(tx, (16,), tw, tb, 1e-5).backward(torch.from_numpy(dz))
    dx, dw, db = blocks.layer_norm_backward(x, w, 1e-5, dz)
    for got, want in ((dx, tx.grad), (dw, tw.grad), (db, tb.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


def test_gelu_tanh_matches_torch():
    import torch
    u = np.linspace(-6, 6, 241)
    tu = torch.tensor(u, requires_grad=True)
    y = torch.nn.functional.gelu(tu, approximate="tanh")
    y.backward(torch.ones_like(tu))
    np.testing.assert_allclose(blocks.gelu_tanh(u), y.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(blocks.gelu_tanh_grad(u), tu.grad.numpy(), rtol=1e-12, atol=1e-14)


def _full_cfg(**kw):
    return _tiny_cfg(full_block=True, drop_q=13107, drop_seed=11, ln_std=0.3, **kw)


@pytest.mark.parametrize("tanh", [False, True])
def test_full_block_step_directional_finite_difference(tanh):
    """Full blocks (LayerNorm, dropout, residual): <grad, v> equals the
    directional derivative of L = <Y_top, G> over the input, every weight and
    the LayerNorm weights (the dropout mask is fixed by its counters)."""
    cfg = _full_cfg(gelu_tanh=tanh)
    inp = _f64_inputs(cfg)
    params = [("x", None)] + [(n, l) for l in range(cfg.n_layers)
                              for n in ("w_in", "b_in", "w_out", "ln_w", "ln_b")]
    gname = {"w_in": "dw_in", "b_in": "db_in", "w_out": "dw_out", "ln_w": "dln_w", "ln_b": "dln_b"}

    def get(i, name, l):
        return getattr(i, name) if l is None else getattr(i, name)[l]

    dirs = {p: RNG.standard_normal(get(inp, *p).shape) for p in params}
    for mode in schedule.MODES:
        out = schedule.run_step(inp, mode)
        analytic = np.sum(out["dX"] * dirs[("x", None)])
        for (n, l), dvec in dirs.items():
            if l is not None:
                analytic += np.sum(out["grads"][l][gname[n]] * dvec)
        eps = 1e-6
        vals = []
        for sgn in (1, -1):
            pert = _f64_inputs(cfg)
            for (n, l), dvec in dirs.items():
                get(pert, n, l)[...] += sgn * eps * dvec
            vals.append(_step_loss(pert))
        fd = (vals[0] - vals[1]) / (2 * eps)
        assert analytic == pytest.approx(fd, rel=1e-7), mode


def test_full_block_schedules_identical_and_residual():
    """All schedules agree bit for bit and match the unsplit reference; with
    zero forward peers and all-zero block weights a full block is the
    identity on the residual stream."""
    cfg = _full_cfg(blocks_=(gen.ATTN, gen.FFN, gen.FFN))
    inp = _f64_inputs(cfg, zero_bwd_peers=False)
    ref = schedule.run_step(inp, "serial_norecompute")
    for mode in schedule.MODES:
        out = schedule.run_step(inp, mode)
        np.testing.assert_array_equal(out["Y"], ref["Y"])
        np.testing.assert_array_equal(out["dX"], ref["dX"])
    unsplit = schedule.run_unsplit(inp)
    np.testing.assert_allclose(ref["Y"], unsplit["Y"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ref["dX"], unsplit["dX"], rtol=1e-12, atol=1e-12)
    for l in range(cfg.n_layers):
        for n in ("dw_in", "db_in", "dw_out", "dln_w", "dln_b"):
            np.testing.assert_allclose(ref["grads"][l][n], unsplit["grads"][l][n], rtol=1e-12, atol=1e-12)
    z = dataclasses.replace(inp, w_out=[np.zeros_like(w) for w in inp.w_out],
                            peers_fwd=np.zeros_like(inp.peers_fwd))
    np.testing.assert_allclose(schedule.run_step(z, "serial_fine")["Y"], inp.x, rtol=0, atol=1e-15)
