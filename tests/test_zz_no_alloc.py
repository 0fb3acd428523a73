"""oases_attention_bwd_noalloc, whose scratch is a static device array,
against oases_attention_bwd with a caller workspace, through the C ABI: the
same dQKV bit for bit on two calls in a row (the second smaller, so it runs
on what the first left in the array), each also checked against the float64
definitions; a problem larger than the static scratch is rejected before
any launch."""
import numpy as np
import pytest

import gen
from oracle import blocks
from helpers import assert_close_local, gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    import torch
    from tensor_model_transformer_tmp_amd import shard
    from tensor_model_transformer_tmp_amd.device import to_device, to_storage


def _bits(rng, shape):
    return gen._f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)).reshape(shape)


def _run(nb, s, nh, d, causal, seed):
    rng = np.random.default_rng(seed)
    a = nh * d
    qkv, dout = _bits(rng, (nb * s, 3 * a)), _bits(rng, (nb * s, a))
    t, do_t = to_device(qkv, gen.BF16, "cuda"), to_device(dout, gen.BF16, "cuda")
    o = torch.empty(nb * s, a, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nb, nh, (s + 63) // 64 * 64, dtype=torch.float32, device="cuda")
    shard.attention_fwd(nb, s, nh, d, causal, t, o, lse)
    want = torch.full((nb * s, 3 * a), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(shard.attention_bwd_workspace_bytes(nb, s, nh), dtype=torch.uint8, device="cuda")
    shard.attention_bwd(nb, s, nh, d, causal, t, o, do_t, lse, want, ws)
    got = torch.full_like(want, float("nan"))
    shard.attention_bwd_noalloc(nb, s, nh, d, causal, t, o, do_t, lse, got)
    torch.cuda.synchronize()
    return qkv, dout, to_storage(got), to_storage(want)


def test_noalloc_matches_workspace_entry_on_two_calls():
    for nb, s, nh, d, causal, seed in ((2, 700, 3, 128, 1, 21), (1, 130, 2, 64, 0, 22)):
        print(f"\n[noalloc nb={nb} s={s} nh={nh} d={d} causal={causal}]", flush=True)
        qkv, dout, got, want = _run(nb, s, nh, d, causal, seed)
        np.testing.assert_array_equal(got, want)
        a = nh * d
        f = gen.bf16_bits_to_f64(qkv)
        q, k, v = (blocks.split_heads(f[:, i * a:(i + 1) * a], nb, s, nh, d) for i in range(3))
        _, p = blocks.attention_fwd(q, k, v, bool(causal))
        dq, dk, dv = blocks.attention_bwd(q, k, v, p, blocks.split_heads(gen.bf16_bits_to_f64(dout), nb, s, nh, d))
        g = gen.bf16_bits_to_f64(got)
        for i, (name, ref) in enumerate((("dQ", dq), ("dK", dk), ("dV", dv))):
            assert_close_local(g[:, i * a:(i + 1) * a], blocks.merge_heads(ref), 2e-2, name, block_cols=d)


def test_noalloc_rejects_problems_beyond_its_scratch():
    need = shard.attention_bwd_workspace_bytes(1, 8192, 1)
    assert need > 48 << 20
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(64, dtype=torch.float32, device="cuda")
    L, ptr = shard.lib(), shard._ptr
    r = L.oases_attention_bwd_noalloc(1, 8192, 1, 64, 1, ptr(x), ptr(x), ptr(x), ptr(lse), ptr(x), None)
    assert r == shard.E_ARG
    assert "static scratch" in L.oases_last_call_error().decode()
    torch.cuda.synchronize()
    assert bool((x == 0).all())
