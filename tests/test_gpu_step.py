"""Whole-step parity on the GPU: every schedule of liboases_shard against the
float64 oracle on the same seeded inputs (1e-5 for float32 storage, 2e-2 for
bf16), bit-identity of the overlapped / graph / serial / default-recompute /
no-recompute schedules, and the per-layer entry points against schedule_step."""
import numpy as np
import pytest

import gen
from oracle import schedule as oschedule
from helpers import assert_close_local, gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    import torch
    from tensor_model_transformer_tmp_amd.device import DeviceShard

MODES = ("overlap_fine", "overlap_fused", "overlap_streams", "serial_fine", "serial_default",
         "serial_norecompute")

# small bf16 stacks with ragged sizes (tokens, hidden, heads and widths that do
# not fill a tile) and both head sizes
SMALL = {
    "pair_d64_ragged": gen.ShardConfig(name="pair_d64_ragged", blocks=(gen.ATTN, gen.FFN),
                                       micro_batch=2, seq=100, hidden=192, heads_per_shard=3,
                                       head_dim=64, ffn_shard=320, tmp_width=3, dtype=gen.BF16,
                                       seed=7),
    "pair_d128": gen.ShardConfig(name="pair_d128", blocks=(gen.ATTN, gen.FFN), micro_batch=4,
                                 seq=160, hidden=256, heads_per_shard=2, head_dim=128,
                                 ffn_shard=512, tmp_width=2, dtype=gen.BF16, seed=8),
    "stack4_d64": gen.ShardConfig(name="stack4_d64", blocks=(gen.ATTN, gen.FFN) * 2,
                                  micro_batch=2, seq=256, hidden=256, heads_per_shard=4,
                                  head_dim=64, ffn_shard=384, tmp_width=4, dtype=gen.BF16,
                                  seed=9),
    "ffn_only_w1": gen.ShardConfig(name="ffn_only_w1", blocks=(gen.FFN,), micro_batch=2, seq=64,
                                   hidden=128, heads_per_shard=1, head_dim=64, ffn_shard=256,
                                   tmp_width=1, dtype=gen.BF16, seed=10),
}


# full transformer blocks (LayerNorm, dropout, residual; tanh GeLU in one of them)
FULL = {
    "full_pair_d64": SMALL["pair_d64_ragged"].with_(name="full_pair_d64", full_block=True, drop_q=6554,
                                                  drop_seed=123),
    "full_pair_d128_tanh": SMALL["pair_d128"].with_(name="full_pair_d128_tanh", full_block=True,
                                                    drop_q=13107, gelu_tanh=True),
    "full_stack4_nodrop": SMALL["stack4_d64"].with_(name="full_stack4_nodrop", full_block=True, drop_q=0),
    # LayerNorm rows held in registers at 8 vectors per lane (hidden 3072), and
    # rows longer than the register form takes (hidden 8256: the multi-pass kernels)
    "full_ffn_h3072": gen.ShardConfig(name="full_ffn_h3072", blocks=(gen.FFN,), micro_batch=2, seq=24,
                                      hidden=3072, heads_per_shard=1, head_dim=64, ffn_shard=192,
                                      tmp_width=2, dtype=gen.BF16, seed=11, full_block=True, drop_q=6554),
    # hidden 4104..8192: rows in registers at 16 vectors per lane (the 8192-hidden
    # full-block workload's LayerNorm kernels), FFN alone and with attention
    "full_ffn_h8192": gen.ShardConfig(name="full_ffn_h8192", blocks=(gen.FFN,), micro_batch=2, seq=16,
                                      hidden=8192, heads_per_shard=1, head_dim=64, ffn_shard=128,
                                      tmp_width=2, dtype=gen.BF16, seed=13, full_block=True, drop_q=6554),
    "full_pair_h8192": gen.ShardConfig(name="full_pair_h8192", blocks=(gen.ATTN, gen.FFN), micro_batch=2,
                                       seq=40, hidden=8192, heads_per_shard=1, head_dim=128, ffn_shard=192,
                                       tmp_width=3, dtype=gen.BF16, seed=14, full_block=True, drop_q=13107),
    "full_ffn_h8256": gen.ShardConfig(name="full_ffn_h8256", blocks=(gen.FFN,), micro_batch=2, seq=16,
                                      hidden=8256, heads_per_shard=1, head_dim=64, ffn_shard=128,
                                      tmp_width=2, dtype=gen.BF16, seed=12, full_block=True, drop_q=6554),
}


def _compare(cfg, got, ref, tol):
    dec = lambda a: gen.storage_to_f64(a, cfg.dtype)
    # whole tensors, elementwise, and per block of 64 rows x 256 columns
    assert_close_local(dec(got["Y"]), ref["Y"], tol, f"{cfg.name} Y", block_cols=256)
    assert_close_local(dec(got["dX"]), ref["dX"], tol, f"{cfg.name} dX", block_cols=256)
    names = ("dw_in", "db_in", "dw_out") + (("dln_w", "dln_b") if cfg.full_block else ())
    for l in range(cfg.n_layers):
        for n in names:
            assert_close_local(got["grads"][l][n], ref["grads"][l][n], tol, f"{cfg.name} layer {l} {n}",
                               block_cols=256)


def _bitwise_equal(a, b):
    np.testing.assert_array_equal(a["Y"], b["Y"])
    np.testing.assert_array_equal(a["dX"], b["dX"])
    for ga, gb in zip(a["grads"], b["grads"]):
        for n in ga:
            np.testing.assert_array_equal(ga[n], gb[n], err_msg=n)


@pytest.mark.parametrize("zero_peers", [False, True])
def test_fp32_ffn_block_all_modes(zero_peers):
    cfg = gen.PRESETS["c1_ffn_fp32"]
    inp = gen.make_inputs(cfg, zero_peers=zero_peers)
    ref = oschedule.run_step(inp, "serial_fine")
    dev = DeviceShard(inp)
    for mode in MODES:
        dev.step(mode)
        _compare(cfg, dev.results(), ref, 1e-5)
    dev.close()


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("zero_peers", [False, True])
def test_bf16_small_stacks(name, zero_peers):
    cfg = SMALL[name]
    inp = gen.make_inputs(cfg, zero_peers=zero_peers)
    ref = oschedule.run_step(inp, "serial_fine")
    dev = DeviceShard(inp)
    dev.step("overlap_fine")
    _compare(cfg, dev.results(), ref, 2e-2)
    dev.close()


@pytest.mark.parametrize("name", ["pair_d64_ragged", "stack4_d64"])
def test_schedules_bit_identical(name):
    cfg = SMALL[name]
    inp = gen.make_inputs(cfg)
    dev = DeviceShard(inp)
    dev.step("serial_fine")
    base = dev.results()
    for mode in MODES:
        for graph in (False, True):
            for _ in range(2):  # graph: first call captures, second replays
                dev.step(mode, use_graph=graph)
                _bitwise_equal(dev.results(), base)
    dev.close()


# sub-batch streams cool-down: from 64 MiB of AllReduce-point inputs
# (T_sb * h * w elements in the storage type) up, sub-batch 1's last weight
# gradients run on sub-batch 0's stream; sized to exactly that much, with
# small blocks around it (float32: FFN only, its column sums by their own kernel)
COOLDOWN = {
    "cool_pair_bf16": gen.ShardConfig(name="cool_pair_bf16", blocks=(gen.ATTN, gen.FFN), micro_batch=2,
                                      seq=1024, hidden=4096, heads_per_shard=1, head_dim=64, ffn_shard=256,
                                      tmp_width=8, dtype=gen.BF16, seed=15),
    "cool_ffn_fp32": gen.ShardConfig(name="cool_ffn_fp32", blocks=(gen.FFN,), micro_batch=2, seq=1024,
                                     hidden=4096, heads_per_shard=1, head_dim=64, ffn_shard=256,
                                     tmp_width=4, dtype=gen.F32, seed=16),
}


@pytest.mark.parametrize("name", list(COOLDOWN))
def test_cooldown_schedule_matches_oracle_and_serial(name):
    """The sub-batch-streams schedule with its cool-down (sub-batch 1's layer-0
    weight gradients on sub-batch 0's stream) against the oracle, and bit for
    bit against the serial schedule, eagerly and as hipGraph replays."""
    cfg = COOLDOWN[name]
    esz = 2 if cfg.dtype == gen.BF16 else 4
    assert (cfg.micro_batch // 2) * cfg.seq * cfg.hidden * cfg.tmp_width * esz >= 64 << 20
    inp = gen.make_inputs(cfg)
    ref = oschedule.run_step(inp, "serial_fine")
    dev = DeviceShard(inp, modes=("overlap_streams", "serial_fine"))
    ops = dev.ctx.schedule_ops("overlap_streams")
    assert ("B_dW", 0, 1, 0) in ops  # the cool-down path is the one taken
    dev.step("serial_fine")
    base = dev.results()
    _compare(cfg, base, ref, 2e-2 if cfg.dtype == gen.BF16 else 1e-5)
    for graph in (False, True):
        for _ in range(2):  # graph: first call captures, second replays
            dev.step("overlap_streams", use_graph=graph)
            _bitwise_equal(dev.results(), base)
    dev.close()


def test_layer_entry_points_match_schedule_step():
    cfg = SMALL["stack4_d64"]
    inp = gen.make_inputs(cfg)
    dev = DeviceShard(inp)
    dev.step("serial_fine")
    base = dev.results()
    L = cfg.n_layers
    for l in range(L):
        for sb in (0, 1):
            dev.ctx.layer_fwd(l, sb)
    for l in reversed(range(L)):
        for sb in (0, 1):
            dev.ctx.layer_bwd_recompute(l, sb)
    dev.ctx.sync()
    _bitwise_equal(dev.results(), base)
    dev.close()


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 9])
@pytest.mark.parametrize("name", ["pair_d64_ragged", "pair_d128"])
def test_attention_variants_full_step(variant, name):
    """Every attention work split (1, 2 or 4 owner waves; single tiles or
    heavy-with-light tile pairs) through the whole step, forward and
    backward, against the oracle with the shard's own outputs visible (zero
    peers)."""
    from tensor_model_transformer_tmp_amd import shard
    cfg = SMALL[name]
    inp = gen.make_inputs(cfg, zero_peers=True)
    ref = oschedule.run_step(inp, "serial_fine")
    shard.set_attention_variant(variant)
    try:
        dev = DeviceShard(inp)
        dev.step("overlap_fine")
        got = dev.results()
        dev.step("serial_norecompute")
        _bitwise_equal(dev.results(), got)
        dev.close()
    finally:
        shard.set_attention_variant(0)
    _compare(cfg, got, ref, 2e-2)


@pytest.mark.parametrize("name", list(FULL))
@pytest.mark.parametrize("zero_peers", [False, True])
def test_full_block_step_matches_oracle(name, zero_peers):
    """Full transformer blocks: every output and gradient (LayerNorm weights
    included) against the oracle, and every schedule, hipGraph replay and the
    per-layer entry points bit-identical to the overlapped step."""
    cfg = FULL[name]
    inp = gen.make_inputs(cfg, zero_peers=zero_peers)
    ref = oschedule.run_step(inp, "serial_fine")
    dev = DeviceShard(inp, modes=MODES)
    dev.step("overlap_fine")
    got = dev.results()
    _compare(cfg, got, ref, 2e-2)
    for mode in MODES:
        for graph in (False, True):
            dev.step(mode, use_graph=graph)
            _bitwise_equal(dev.results(), got)
    L = cfg.n_layers
    for l in range(L):
        for sb in (0, 1):
            dev.ctx.layer_fwd(l, sb)
    for l in reversed(range(L)):
        for sb in (0, 1):
            dev.ctx.layer_bwd_recompute(l, sb)
    dev.ctx.sync()
    _bitwise_equal(dev.results(), got)
    dev.close()


def test_event_timeline_of_overlapped_steps():
    """oases_profile_timeline over two eager sub-batch-stream steps: one entry
    per kernel-class launch of the op list, on both streams, each ending after
    it starts; the step's result is the same as without the events."""
    cfg = SMALL["pair_d128"]
    dev = DeviceShard(gen.make_inputs(cfg), device="cuda", modes=("overlap_streams",))
    try:
        dev.ctx.schedule_step("overlap_streams", False)
        torch.cuda.synchronize()
        y0 = dev.y.clone()
        dev.ctx.profile_begin("all", 1024)
        for _ in range(2):
            dev.ctx.schedule_step("overlap_streams", False)
        rows = dev.ctx.profile_timeline(1024)
        per_step = len(rows) // 2
        assert len(rows) == 2 * per_step and per_step > 0
        kinds = {r[0] for r in rows}
        assert {"gemm_fwd", "gemm_dx", "gemm_dw", "attn_fwd", "attn_bwd", "sum"} <= kinds
        assert {r[1] for r in rows} == {0, 1}
        assert all(b >= a >= 0.0 for _, _, a, b in rows)
        # C(F) and C(B) of each layer and sub-batch, two steps
        assert sum(1 for r in rows if r[0] == "sum") == 2 * 4 * cfg.n_layers
        assert torch.equal(dev.y, y0)
        # a second run with too small a buffer is an argument error and keeps the run open
        dev.ctx.profile_begin("all", 1024)
        dev.ctx.schedule_step("overlap_streams", False)
        with pytest.raises(Exception):
            dev.ctx.profile_timeline(1)
        assert len(dev.ctx.profile_timeline(1024)) == per_step
    finally:
        dev.close()
