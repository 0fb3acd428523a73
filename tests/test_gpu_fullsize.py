"""Parity at the full workload sizes, in the launch configuration bench.py
times (overlapped fine-grained schedule, eager on two streams, and the fused
overlap in which the sums run on the next GEMM launch; automatic tile and
kernel-layout choice), against the complete float64 oracle step on the
same seeded inputs: every element of Y, dX and every weight / bias gradient.

Each workload runs twice: with the seeded peers, as timed, and with zero
peer partials, so the shard's own outputs (P and dX_own) are also compared
without being masked by the N(0,1) peers.  The hipGraph
replay and the serial schedule must reproduce the overlapped result bit for
bit at full size."""
import numpy as np
import pytest

import gen
from oracle import schedule as oschedule, sums
from helpers import assert_close_local, gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    import torch
    from tensor_model_transformer_tmp_amd import shard
    from tensor_model_transformer_tmp_amd.device import DeviceShard, to_device, to_storage

TOL = 2e-2

CASES = [("c2_pair_h1024", False), ("c2_pair_h1024", True), ("c3_pair_h4096", False),
         ("c3_pair_h4096", True), ("c4_stack8_h2048", False), ("c4_stack8_h2048", True),
         ("c5_pair_h8192", False), ("c5_pair_h8192", True),
         ("c2_full_h1024", False), ("c2_full_h1024", True), ("c5_full_h8192", False), ("c5_full_h8192", True)]


def _compare(cfg, got, ref):
    dec = lambda a: gen.storage_to_f64(a, cfg.dtype)
    # whole tensors, elementwise, and per block of 64 rows x 256 columns
    assert_close_local(dec(got["Y"]), ref["Y"], TOL, f"{cfg.name} Y", block_cols=256)
    assert_close_local(dec(got["dX"]), ref["dX"], TOL, f"{cfg.name} dX", block_cols=256)
    names = ("dw_in", "db_in", "dw_out") + (("dln_w", "dln_b") if cfg.full_block else ())
    for l in range(cfg.n_layers):
        for n in names:
            assert_close_local(got["grads"][l][n], ref["grads"][l][n], TOL, f"{cfg.name} layer {l} {n}",
                               block_cols=256)


def _bitwise_equal(a, b, what):
    np.testing.assert_array_equal(a["Y"], b["Y"], err_msg=what)
    np.testing.assert_array_equal(a["dX"], b["dX"], err_msg=what)
    for ga, gb in zip(a["grads"], b["grads"]):
        for n in ga:
            np.testing.assert_array_equal(ga[n], gb[n], err_msg=f"{what} {n}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,zero_peers", CASES)
def test_full_size_step_matches_oracle(name, zero_peers):
    cfg = gen.PRESETS[name] if name in gen.PRESETS else gen.FULL_PRESETS[name]
    inp = gen.make_inputs(cfg, zero_peers=zero_peers)
    print(f"\n[{name} zero_peers={zero_peers}] device step", flush=True)
    dev = DeviceShard(inp, modes=("overlap_fine", "overlap_fused", "overlap_streams", "serial_fine"))
    dev.step("overlap_fine", use_graph=False)
    got = dev.results()
    for mode, graph in (("overlap_fine", True), ("overlap_fine", True), ("overlap_fused", False),
                        ("overlap_fused", True), ("overlap_fused", True), ("overlap_streams", False),
                        ("overlap_streams", True), ("overlap_streams", True), ("serial_fine", False)):
        dev.step(mode, use_graph=graph)
        _bitwise_equal(dev.results(), got, f"{name} {mode} graph={graph}")
    dev.close()
    del dev
    torch.cuda.empty_cache()
    print(f"[{name}] oracle step", flush=True)
    ref = oschedule.run_step(inp, "serial_fine")
    _compare(cfg, got, ref)


@pytest.mark.parametrize("name", ["c3_pair_h4096", "c5_pair_h8192"])
def test_full_size_allreduce_point_bit_exact(name):
    """One AllReduce point at the workload's full size (T_sb x h elements,
    w-1 peers) in the launch configuration of the step."""
    cfg = gen.PRESETS[name]
    n = cfg.t_sb * cfg.hidden
    w1 = cfg.tmp_width - 1
    rng = np.random.default_rng(cfg.seed)
    own = gen._f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    peers = gen._f32_to_bf16_bits(rng.standard_normal(w1 * n).astype(np.float32)).reshape(w1, n)
    t_own, t_peers = to_device(own, gen.BF16, "cuda"), to_device(peers, gen.BF16, "cuda")
    out = torch.empty_like(t_own)
    shard.allreduce_point(gen.BF16, t_own, t_peers, w1, out)
    torch.cuda.synchronize()
    want = sums.allreduce_point_storage(own, [peers[k] for k in range(w1)], True)
    np.testing.assert_array_equal(to_storage(out), want)
