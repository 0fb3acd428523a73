"""Seeded input generator: determinism, shapes and the bf16 rounding of drawn values."""
import numpy as np

import gen


def test_presets_shapes():
    c = gen.PRESETS["c3_pair_h4096"]
    assert c.t_sb == 2048 and c.attn_width == 512 and c.n_in(0) == 1536 and c.n_in(1) == 2048
    assert c.n_mid(0) == 512 and c.n_mid(1) == 2048
    assert gen.PRESETS["c1_ffn_fp32"].t_sb == 32
    assert gen.PRESETS["c4_stack8_h2048"].n_layers == 8
    assert [gen.PRESETS[n].seed for n in gen.PRESET_ORDER] == [20250625 + i for i in range(5)]


def test_deterministic_and_distinct():
    cfg = gen.PRESETS["c1_ffn_fp32"]
    a, b = gen.make_inputs(cfg), gen.make_inputs(cfg)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.peers_bwd, b.peers_bwd)
    assert not np.array_equal(a.peers_fwd[0, 0, 0], a.peers_fwd[0, 1, 0])
    assert not np.array_equal(a.peers_fwd, a.peers_bwd)
    assert np.all(a.b_in[0] == 0)
    assert abs(a.w_in[0].std() - 0.02) < 0.002 and abs(a.x.std() - 1) < 0.05
    z = gen.make_inputs(cfg, zero_peers=True)
    assert not z.peers_fwd.any() and not z.peers_bwd.any()
    np.testing.assert_array_equal(z.x, a.x)


def test_bf16_storage_round_to_nearest_even():
    cfg = gen.PRESETS["c2_pair_h1024"].with_(micro_batch=2, seq=8)
    inp = gen.make_inputs(cfg, zero_peers=True)
    assert inp.x.dtype == np.uint16
    vals = inp.f64("x")
    # every stored value is a bf16 number: its float32 pattern has 16 zero low bits
    assert np.all((vals.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    # and it is the nearest bf16 to the float32 draw
    rng = np.random.default_rng([cfg.seed, gen.K_X, 0, 0, 0])
    v32 = rng.standard_normal(cfg.tokens * cfg.hidden).astype(np.float32)
    err = np.abs(vals.ravel() - v32.astype(np.float64))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(v32.astype(np.float64)))) - 7)
    assert np.all(err <= ulp / 2)
    # ties go to the even mantissa: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert gen._f32_to_bf16_bits(np.array([1 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert gen._f32_to_bf16_bits(np.array([1 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82
