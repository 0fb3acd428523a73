"""Single-kernel parity on the GPU: the AllReduce-point sum (bit-exact against
the storage-type oracle), the forward GEMM with bias / GeLU epilogues, and
causal attention forward, against float64 definitions on the same inputs."""
import math

import numpy as np
import pytest

import gen
from oracle import blocks, sums
from helpers import assert_close, assert_close_local, gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    import torch
    from tensor_model_transformer_tmp_amd import shard
    from tensor_model_transformer_tmp_amd.device import to_device, to_storage


def _bf16_bits(rng, shape, std=1.0):
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    return gen._f32_to_bf16_bits(v).reshape(shape)


@pytest.mark.parametrize("form", [1, 2])
@pytest.mark.parametrize("dtype", [gen.BF16, gen.F32])
@pytest.mark.parametrize("n,n_peers", [(8, 1), (4096 * 8 + 24, 0), (4096 * 8 + 24, 3), (4096 * 8 + 24, 5),
                                        (1 << 20, 7), (3 * 2048 * 1024, 3)])
def test_allreduce_point_bit_exact(dtype, n, n_peers, form):
    """Both forms of the sum kernel (several vectors per thread in flight, or
    one) against the float32 sequential sum, bit for bit."""
    rng = np.random.default_rng(n + n_peers)
    mk = (lambda s: _bf16_bits(rng, s)) if dtype == gen.BF16 else \
        (lambda s: rng.standard_normal(s).astype(np.float32))
    own = mk((n,))
    peers = mk((max(n_peers, 1), n))
    dev = "cuda"
    t_own, t_peers = to_device(own, dtype, dev), to_device(peers, dtype, dev)
    out = torch.empty_like(t_own)
    shard.set_sum_variant(form)
    try:
        shard.allreduce_point(dtype, t_own, t_peers, n_peers, out)
        torch.cuda.synchronize()
    finally:
        shard.set_sum_variant(0)
    want = sums.allreduce_point_storage(own, [peers[k] for k in range(n_peers)], dtype == gen.BF16)
    np.testing.assert_array_equal(to_storage(out), want)


@pytest.mark.parametrize("m,n,k", [(200, 192, 128), (1000, 520, 576), (2048, 1024, 1024),
                                   (4096, 3072, 512), (37, 8, 8)])
@pytest.mark.parametrize("epi", ["store", "bias", "gelu", "gelu_tanh"])
def test_gemm_fwd_bf16(m, n, k, epi):
    rng = np.random.default_rng(m * 7 + n + k)
    a, w = _bf16_bits(rng, (m, k)), _bf16_bits(rng, (n, k), 0.05)
    b = _bf16_bits(rng, (n,), 0.5)
    dev = "cuda"
    ta, tw, tb = (to_device(x, gen.BF16, dev) for x in (a, w, b))
    c = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    pre = torch.empty_like(c) if epi.startswith("gelu") else None
    if epi == "gelu_tanh":
        shard.gemm(shard.BF16, ta, tw, c, 0, 0, "gelu_tanh", bias=tb, pre=pre)
    else:
        shard.gemm_fwd(shard.BF16, ta, tw, c, bias=None if epi == "store" else tb,
                       gelu=epi == "gelu", pre=pre)
    torch.cuda.synchronize()
    af, wf, bf = (gen.bf16_bits_to_f64(x) for x in (a, w, b))
    ref = af @ wf.T + (0 if epi == "store" else bf)
    if epi.startswith("gelu"):
        assert_close(gen.bf16_bits_to_f64(to_storage(pre)), ref, 8e-3, "pre-activation")
        ref = blocks.gelu_tanh(ref) if epi == "gelu_tanh" else blocks.gelu(ref)
    got = gen.bf16_bits_to_f64(to_storage(c))
    assert_close(got, ref, 8e-3, f"C {m}x{n}x{k} {epi}")
    np.testing.assert_allclose(got, ref, rtol=1.6e-2, atol=1e-2 * np.abs(ref).max())


def test_gemm_fwd_f32():
    rng = np.random.default_rng(5)
    m, n, k = 77, 136, 64
    a = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    ta, tw, tb = (torch.from_numpy(x).cuda() for x in (a, w, b))
    c, pre = torch.empty(m, n, device="cuda"), torch.empty(m, n, device="cuda")
    shard.gemm_fwd(shard.F32, ta, tw, c, bias=tb, gelu=True, pre=pre)
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T + b
    assert_close(pre.cpu().numpy(), ref, 1e-6, "pre")
    assert_close(c.cpu().numpy(), blocks.gelu(ref), 1e-6, "gelu")


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nb,s,nh,causal", [(1, 1, 1, True), (2, 100, 3, True), (1, 300, 2, False),
                                            (2, 512, 2, True), (1, 1030, 1, True)])
def test_attention_fwd(variant, d, nb, s, nh, causal):
    rng = np.random.default_rng(d + s + nh)
    a = nh * d
    qkv = _bf16_bits(rng, (nb * s, 3 * a))
    t = to_device(qkv, gen.BF16, "cuda")
    o = torch.empty(nb * s, a, dtype=torch.bfloat16, device="cuda")
    s_pad = (s + 63) // 64 * 64
    lse = torch.empty(nb, nh, s_pad, dtype=torch.float32, device="cuda")
    shard.set_attention_variant(variant)
    try:
        shard.attention_fwd(nb, s, nh, d, causal, t, o, lse)
        torch.cuda.synchronize()
    finally:
        shard.set_attention_variant(0)
    f = gen.bf16_bits_to_f64(qkv)
    q, k, v = (blocks.split_heads(f[:, i * a:(i + 1) * a], nb, s, nh, d) for i in range(3))
    o_ref, _ = blocks.attention_fwd(q, k, v, causal)
    assert_close_local(gen.bf16_bits_to_f64(to_storage(o)), blocks.merge_heads(o_ref), 2e-2, "O",
                       block_cols=d)
    sc = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d)
    if causal:
        sc = np.where(np.triu(np.ones((s, s), bool), 1), -np.inf, sc)
    mx = sc.max(-1, keepdims=True)
    lse_ref = (mx + np.log(np.exp(sc - mx).sum(-1, keepdims=True)))[..., 0]
    np.testing.assert_allclose(lse.cpu().numpy()[..., :s], lse_ref, rtol=0, atol=2e-3)


GEMM_SHAPES = [(200, 192, 128), (1000, 520, 576), (2048, 1024, 1024), (296, 136, 200), (64, 8, 64)]


@pytest.mark.parametrize("variant", list(range(23)))
@pytest.mark.parametrize("kind", ["fwd", "dx", "dx_gelu", "dx_gelu_tanh", "dw", "dw_colsum"])
@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_layouts_and_tiles(variant, kind, m, n, k):
    """Every operand layout / epilogue of the step's GEMMs and every tile
    configuration, against a float64 product of the same bf16 operands."""
    rng = np.random.default_rng(m + 3 * n + 7 * k + variant)
    dev = "cuda"
    shard.set_gemm_tile_variant(variant)
    try:
        a_km = _bf16_bits(rng, (m, k))          # A(m, k), stored [M][K]
        b_nk = _bf16_bits(rng, (n, k), 0.05)    # B(k, n) stored [N][K]
        af = gen.bf16_bits_to_f64(a_km)
        bf = gen.bf16_bits_to_f64(b_nk)
        ref = af @ bf.T
        if kind == "fwd":
            c = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            shard.gemm(shard.BF16, to_device(a_km, gen.BF16, dev), to_device(b_nk, gen.BF16, dev), c,
                       0, 0, "store")
        elif kind.startswith("dx"):
            b_kn = np.ascontiguousarray(b_nk.T)  # stored [K][N] (n contiguous)
            c = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            aux = None
            if kind.startswith("dx_gelu"):
                u = _bf16_bits(rng, (m, n))
                aux = to_device(u, gen.BF16, dev)
                grad = blocks.gelu_tanh_grad if kind == "dx_gelu_tanh" else blocks.gelu_grad
                ref = ref * grad(gen.bf16_bits_to_f64(u))
            epi = {"dx": "store", "dx_gelu": "gelu_bwd", "dx_gelu_tanh": "gelu_tanh_bwd"}[kind]
            shard.gemm(shard.BF16, to_device(a_km, gen.BF16, dev), to_device(b_kn, gen.BF16, dev), c,
                       0, 1, epi, m=m, n=n, k=k, aux=aux)
        else:
            a_mk = np.ascontiguousarray(a_km.T)  # stored [K][M] (m contiguous)
            b_kn = np.ascontiguousarray(b_nk.T)
            old = rng.standard_normal((m, n)).astype(np.float32)
            c = torch.from_numpy(old).to(dev)
            cs = None
            if kind == "dw_colsum":   # plus the sums of A over k, added to old values
                old_cs = rng.standard_normal(m).astype(np.float32)
                cs = torch.from_numpy(old_cs).to(dev)
            shard.gemm(shard.BF16, to_device(a_mk, gen.BF16, dev), to_device(b_kn, gen.BF16, dev), c,
                       1, 1, "f32_colsum" if cs is not None else "f32", m=m, n=n, k=k, pre=cs, beta=1)
            ref = ref + old
        torch.cuda.synchronize()
        got = c.cpu().numpy() if c.dtype == torch.float32 else gen.bf16_bits_to_f64(to_storage(c))
        tol = 1e-5 if kind.startswith("dw") else 8e-3
        assert_close(got, ref, tol, f"{kind} {m}x{n}x{k} variant {variant}")
        if kind == "dw_colsum":
            assert_close(cs.cpu().numpy(), af.sum(axis=1) + old_cs, 1e-5,
                         f"column sums {m}x{n}x{k} variant {variant}")
    finally:
        shard.set_gemm_tile_variant(0)


@pytest.mark.parametrize("variant", [0, 3, 4, 5, 14, 20])
def test_gemm_empty_k(variant):
    """k = 0: the product is zero, so C is the epilogue of zero -- the bias
    (forward), zeros (data gradient), and the old float32 C (weight gradient
    accumulating with beta) -- and no operand is read (the operand pointers
    here are small buffers of the wrong size)."""
    m, n = 200, 136
    dev = "cuda"
    shard.set_gemm_tile_variant(variant)
    try:
        rng = np.random.default_rng(variant)
        wide_a = torch.zeros(1, 208, dtype=torch.bfloat16, device=dev)  # m-contiguous stride >= m
        wide_b = torch.zeros(1, 136, dtype=torch.bfloat16, device=dev)  # n-contiguous stride >= n
        narrow = torch.zeros(2, 8, dtype=torch.bfloat16, device=dev)    # k-contiguous stride 8 >= k
        bias_bits = _bf16_bits(rng, (n,))
        bias = to_device(bias_bits, gen.BF16, dev)
        c = torch.full((m, n), float("nan"), device=dev).to(torch.bfloat16)
        shard.gemm(shard.BF16, narrow, narrow, c, 0, 0, "bias", m=m, n=n, k=0, bias=bias)
        dxc = torch.full((m, n), float("nan"), device=dev).to(torch.bfloat16)
        shard.gemm(shard.BF16, narrow, wide_b, dxc, 0, 1, "store", m=m, n=n, k=0)
        old = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).to(dev)
        dwc = old.clone()
        shard.gemm(shard.BF16, wide_a, wide_b, dwc, 1, 1, "f32", m=m, n=n, k=0, beta=1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_storage(c), np.broadcast_to(bias_bits, (m, n)))
        np.testing.assert_array_equal(to_storage(dxc), np.zeros((m, n), np.uint16))
        np.testing.assert_array_equal(dwc.cpu().numpy(), old.cpu().numpy())
    finally:
        shard.set_gemm_tile_variant(0)


def test_mfma_probe_runs():
    """The MFMA throughput probe issues its MFMAs (finite, nonzero per-lane
    checksums) and reports the FLOPs of its launch."""
    out = torch.zeros(2 * 256, dtype=torch.float32, device="cuda")
    flop = shard.mfma_probe(2, 3, out)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert flop == 2 * 4 * 4 * 3 * 32 * 32 * 16 * 2
    assert np.isfinite(v).all() and (v != 0).any()


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nb,s,nh,causal", [(1, 1, 1, True), (2, 100, 3, True), (1, 300, 2, False),
                                            (2, 512, 2, True), (1, 1030, 1, True), (1, 130, 2, False)])
def test_attention_bwd(variant, d, nb, s, nh, causal):
    """dQ, dK and dV of the attention backward (delta, dK/dV with dS, dQ from
    dS) against the float64 definitions, per head and per 64-row block, with
    O and lse from the GPU forward (both sides see the same bf16 O)."""
    rng = np.random.default_rng(3 * d + s + 7 * nh + variant)
    a = nh * d
    qkv = _bf16_bits(rng, (nb * s, 3 * a))
    dout = _bf16_bits(rng, (nb * s, a))
    t = to_device(qkv, gen.BF16, "cuda")
    do_t = to_device(dout, gen.BF16, "cuda")
    o = torch.empty(nb * s, a, dtype=torch.bfloat16, device="cuda")
    s_pad = (s + 63) // 64 * 64
    lse = torch.empty(nb, nh, s_pad, dtype=torch.float32, device="cuda")
    dqkv = torch.full((nb * s, 3 * a), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((shard.attention_bwd_workspace_bytes(nb, s, nh),), 255, dtype=torch.uint8, device="cuda")
    shard.set_attention_variant(variant)
    try:
        shard.attention_fwd(nb, s, nh, d, causal, t, o, lse)
        shard.attention_bwd(nb, s, nh, d, causal, t, o, do_t, lse, dqkv, ws)
        torch.cuda.synchronize()
    finally:
        shard.set_attention_variant(0)
    f = gen.bf16_bits_to_f64(qkv)
    q, k, v = (blocks.split_heads(f[:, i * a:(i + 1) * a], nb, s, nh, d) for i in range(3))
    _, p = blocks.attention_fwd(q, k, v, causal)
    dof = blocks.split_heads(gen.bf16_bits_to_f64(dout), nb, s, nh, d)
    dq, dk, dv = blocks.attention_bwd(q, k, v, p, dof)
    got = gen.bf16_bits_to_f64(to_storage(dqkv))
    for i, (name, ref) in enumerate((("dQ", dq), ("dK", dk), ("dV", dv))):
        assert_close_local(got[:, i * a:(i + 1) * a], blocks.merge_heads(ref), 2e-2, name, block_cols=d)


def test_attention_bwd_rejects_bad_arguments():
    dev = "cuda"
    x = torch.zeros(64, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(64, dtype=torch.float32, device=dev)
    need = shard.attention_bwd_workspace_bytes(1, 8, 1)
    small = torch.zeros(need - 16, dtype=torch.uint8, device=dev)
    L = shard.lib()
    ptr = shard._ptr
    assert L.oases_attention_bwd(1, 8, 1, 96, 1, ptr(x), ptr(x), ptr(x), ptr(lse), ptr(x), ptr(small), need, None) \
        == shard.E_ARG
    assert L.oases_attention_bwd(1, 8, 1, 64, 1, ptr(x), ptr(x), ptr(x), ptr(lse), ptr(x), ptr(small),
                                 need - 16, None) == shard.E_ARG
    assert "need" in L.oases_last_call_error().decode()
