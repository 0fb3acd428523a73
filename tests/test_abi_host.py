"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, validates configurations, buffers and call
order before touching HIP, and issues the same op lists as the oracle's
schedules."""
import ctypes
import os
import re

import pytest

import gen
from oracle import schedule as oschedule
from tensor_model_transformer_tmp_amd import shard

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "oases_shard.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_library_exports_every_declared_symbol():
    lib = shard.lib()
    declared = _declared_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(shard.EXPORTED)


def _cfg(**kw):
    return gen.PRESETS["c2_pair_h1024"].with_(**kw)


def test_mfma_probe_validation():
    L = shard.lib()
    assert L.oases_mfma_probe(0, 1, None, None) == shard.E_ARG
    assert L.oases_mfma_probe(1, 0, None, None) == shard.E_ARG
    assert L.oases_mfma_probe(1, 1, None, None) == shard.E_ARG


def test_profile_timeline_validation():
    L = shard.lib()
    n = ctypes.c_int32(0)
    assert L.oases_profile_timeline(None, 0, None, None, None, None, ctypes.byref(n)) == shard.E_ARG


def test_create_validation():
    for bad, code in ((dict(micro_batch=3), shard.E_SHAPE), (dict(micro_batch=0), shard.E_SHAPE),
                      (dict(hidden=100), shard.E_SHAPE), (dict(head_dim=96), shard.E_SHAPE),
                      (dict(ffn_shard=65), shard.E_SHAPE), (dict(tmp_width=0), shard.E_SHAPE),
                      (dict(dtype=gen.F32), shard.E_UNSUPPORTED), (dict(dtype=7), shard.E_ARG),
                      (dict(blocks=(0, 5)), shard.E_ARG), (dict(blocks=()), shard.E_SHAPE)):
        with pytest.raises(shard.OasesError) as ei:
            shard.ShardContext(_cfg(**bad))
        assert ei.value.code == code, bad
    # fp32 FFN-only stacks are supported
    shard.ShardContext(gen.PRESETS["c1_ffn_fp32"]).close()
    # full transformer blocks: bf16 only, drop_q in [0, 65535], eps > 0
    full = dict(full_block=True, drop_q=6554)
    for bad, code in ((dict(drop_q=65536), shard.E_ARG), (dict(drop_q=-1), shard.E_ARG),
                      (dict(ln_eps=0.0), shard.E_ARG)):
        with pytest.raises(shard.OasesError) as ei:
            shard.ShardContext(_cfg(**{**full, **bad}))
        assert ei.value.code == code, bad
    for cfg in (gen.PRESETS["c1_ffn_fp32"].with_(full_block=True),
                gen.PRESETS["c1_ffn_fp32"].with_(gelu_tanh=True)):
        with pytest.raises(shard.OasesError) as ei:
            shard.ShardContext(cfg)
        assert ei.value.code == shard.E_UNSUPPORTED
    shard.ShardContext(_cfg(**full, gelu_tanh=True)).close()


def test_workspace_bytes_modes():
    cfg = gen.PRESETS["c4_stack8_h2048"]
    fine = shard.workspace_bytes(cfg, "serial_fine")
    assert shard.workspace_bytes(cfg, "overlap_fine") == fine
    assert shard.workspace_bytes(cfg, "serial_default") > fine
    assert shard.workspace_bytes(cfg, "serial_norecompute") > 4 * fine // 3
    assert fine % 256 == 0


def _fake_buffers(cfg, align=256, ws=None):
    """Aligned host addresses that the library never dereferences on the host."""
    base = 1 << 32
    addrs = iter(range(base, base + 64 * (1 << 20), 1 << 20))
    b = shard.Buffers(*[next(addrs) for _ in range(8)],
                      ws if ws is not None else shard.workspace_bytes(cfg, "serial_fine"))
    params = (shard.LayerParams * cfg.n_layers)()
    for l in range(cfg.n_layers):
        params[l] = shard.LayerParams(*[next(addrs) for _ in range(6)])
    return b, params


def test_bind_validation_and_call_order():
    cfg = _cfg()
    ctx = shard.ShardContext(cfg)
    b, p = _fake_buffers(cfg)
    # call order before bind
    assert ctx.status("layer_fwd", 0, 0) == shard.E_STATE
    assert ctx.status("schedule_step", 0, 0) == shard.E_STATE
    # argument checks
    assert ctx.status("layer_fwd", 2, 0) == shard.E_ARG
    assert ctx.status("layer_fwd", 0, 2) == shard.E_ARG
    assert ctx.status("layer_bwd_recompute", -1, 0) == shard.E_ARG
    assert ctx.status("schedule_step", 9, 0) == shard.E_ARG
    bad = shard.Buffers.from_buffer_copy(b)
    bad.x = None
    assert ctx.bind_raw(bad, p) == shard.E_ARG
    bad = shard.Buffers.from_buffer_copy(b)
    bad.dy = b.dy + 8
    assert ctx.bind_raw(bad, p) == shard.E_ALIGN
    bad = shard.Buffers.from_buffer_copy(b)
    bad.workspace = b.workspace + 16
    assert ctx.bind_raw(bad, p) == shard.E_ALIGN
    bad = shard.Buffers.from_buffer_copy(b)
    bad.workspace_bytes = 1024
    assert ctx.bind_raw(bad, p) == shard.E_ARG
    p2 = (shard.LayerParams * cfg.n_layers)(*p)
    p2[1].db_in = None
    assert ctx.bind_raw(b, p2) == shard.E_ARG
    assert "layer 1 db_in" in ctx.last_error()
    assert ctx.bind_raw(b, p) == shard.OK
    # state machine: backward before forward, skipped layers, sub-batch order
    assert ctx.status("layer_bwd_recompute", 1, 0) == shard.E_STATE
    assert "before the forward" in ctx.last_error()
    assert ctx.status("layer_fwd", 1, 0) == shard.E_STATE
    # streams are not set, so the first legal call stops there, before any HIP work
    assert ctx.status("layer_fwd", 0, 0) == shard.E_STATE
    assert "streams" in ctx.last_error()
    ctx.close()


def test_single_kernel_entry_validation():
    L = shard.lib()
    assert L.oases_allreduce_point(1, 16, 32, 10, 1, 48, 12, None) == shard.E_ARG  # n % 8
    assert L.oases_allreduce_point(1, 17, 32, 16, 1, 48, 16, None) == shard.E_ALIGN
    assert L.oases_allreduce_point(1, 16, 32, 16, 1, 48, 0, None) == shard.OK  # empty
    # n % 8 != 0
    assert L.oases_gemm(1, 0, 0, 0, 4, 12, 16, 16, 16, 32, 16, 48, 16, None, None, None, 0, 0,
                        None) == shard.E_ARG
    # unsupported layout / epilogue pair
    assert L.oases_gemm(1, 1, 1, 0, 4, 16, 16, 16, 16, 32, 16, 48, 16, None, None, None, 0, 0,
                        None) == shard.E_UNSUPPORTED
    # bias epilogue without a bias
    assert L.oases_gemm(1, 0, 0, 1, 4, 16, 16, 16, 16, 32, 16, 48, 16, None, None, None, 0, 0,
                        None) == shard.E_ARG
    # column-sum epilogue: bfloat16 only, needs its float32 output in pre
    assert L.oases_gemm(0, 1, 1, 5, 4, 16, 16, 16, 16, 32, 16, 48, 16, None, 64, None, 0, 0,
                        None) == shard.E_UNSUPPORTED
    assert L.oases_gemm(1, 1, 1, 5, 4, 16, 16, 16, 16, 32, 16, 48, 16, None, None, None, 0, 0,
                        None) == shard.E_ARG
    # empty problem is a no-op
    assert L.oases_gemm(1, 0, 0, 0, 0, 16, 16, 16, 16, 32, 16, 48, 16, None, None, None, 0, 0,
                        None) == shard.OK
    assert L.oases_gemm_tile_variant(23) == shard.E_ARG
    assert L.oases_attention_variant(10) == shard.E_ARG
    assert L.oases_attention_variant(-1) == shard.E_ARG
    assert L.oases_attention_fwd(1, 8, 1, 96, 1, 16, 32, 48, None) == shard.E_ARG


@pytest.mark.parametrize("n_layers", [1, 2, 5, 8])
def test_op_lists_match_oracle_schedules(n_layers):
    cfg = _cfg(blocks=tuple(i % 2 for i in range(n_layers)))
    ctx = shard.ShardContext(cfg)
    for mode in oschedule.MODES:
        assert ctx.schedule_ops(mode) == oschedule.build_ops(n_layers, mode), mode
    # the fused overlap runs the overlapped op list (sums on the next GEMM launch)
    assert ctx.schedule_ops("overlap_fused") == oschedule.build_ops(n_layers, "overlap_fine")
    # one stream per sub-batch: the same ops in the same order, stream =
    # sub-batch (at this size, 16 MiB of AllReduce-point inputs, the
    # cool-down keeps every op on its sub-batch's stream)
    by_sb = [(k, l, sb, sb) for (k, l, sb, _) in oschedule.build_ops(n_layers, "overlap_fine")]
    assert ctx.schedule_ops("overlap_streams") == by_sb
    ctx.close()


@pytest.mark.parametrize("preset,moved", [("c2_pair_h1024", False), ("c3_pair_h4096", True),
                                          ("c4_stack8_h2048", True), ("c5_pair_h8192", True),
                                          ("c1_ffn_fp32", False)])
def test_cooldown_stream_of_last_weight_gradients(preset, moved):
    """Sub-batch streams: from 64 MiB of AllReduce-point inputs up, sub-batch
    1's last weight gradients (B_dW of layer 0) run on sub-batch 0's stream."""
    cfg = gen.PRESETS[preset]
    ctx = shard.ShardContext(cfg)
    ops = ctx.schedule_ops("overlap_streams")
    want = [(k, l, sb, 0 if moved and (k, l) == ("B_dW", 0) else sb)
            for (k, l, sb, _) in oschedule.build_ops(cfg.n_layers, "overlap_fine")]
    assert ops == want
    # the other modes never move it
    assert ctx.schedule_ops("overlap_fine") == oschedule.build_ops(cfg.n_layers, "overlap_fine")
    ctx.close()
