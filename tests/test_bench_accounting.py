"""Host checks of bench.py's counted work and its command-line contract (no GPU)."""
import os
import subprocess
import sys

import pytest

import bench
import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# counted GFLOP per step (forward / recompute / backward), worked out by hand
# from the workload sizes to three significant figures: 2MNK per executed
# GEMM (the recompute skips the dead row-parallel GEMM) and the causal lower
# triangle for attention
EXPECTED_GFLOP = {
    "c2_pair_h1024": (26.9, 16.1, 53.7),
    "c3_pair_h4096": (210, 125, 421),
    "c4_stack8_h2048": (859, 515, 1718),
    "c5_pair_h8192": (842, 498, 1684),
}


@pytest.mark.parametrize("name", list(EXPECTED_GFLOP))
def test_step_flops_match_the_workload_sizes(name):
    got = [x / 1e9 for x in bench.step_flops(gen.PRESETS[name])]
    for g, e in zip(got, EXPECTED_GFLOP[name]):
        assert abs(g - e) / e < 5e-3, (name, got)


def test_attention_counts_the_lower_triangle():
    cfg = gen.PRESETS["c2_pair_h1024"]
    s, d = cfg.seq, cfg.head_dim
    per_head = 2.0 * s * (s + 1) / 2 * d
    assert bench.attn_matmul_flops(cfg) == per_head * (cfg.micro_batch // 2) * cfg.heads_per_shard


@pytest.mark.parametrize("name", list(EXPECTED_GFLOP))
def test_class_work_adds_up_to_the_step(name):
    cfg = gen.PRESETS[name]
    total = sum(bench.class_work(cfg, k)[0] for k in ("gemm_fwd", "gemm_dx", "gemm_dw", "attn_fwd", "attn_bwd"))
    assert abs(total - sum(bench.step_flops(cfg))) <= 1e-9 * total


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_power_summary_takes_readings_inside_the_window():
    rows = [{"t": 0.0, "t_done": 0.5, "power_w": 250.0, "gfx_mhz": [100, 100]},     # idle, before
            {"t": 10.2, "t_done": 10.8, "power_w": 1300.0, "gfx_mhz": [1900, 1880]},  # first second: skipped
            {"t": 11.2, "t_done": 11.8, "power_w": 1350.0, "gfx_mhz": [1850, 1870]},
            {"t": 11.9, "t_done": 12.5, "power_w": 1370.0, "gfx_mhz": [1810, 1830]},
            {"t": 13.7, "t_done": 14.3, "power_w": 900.0, "gfx_mhz": [2400, 2400]}]   # ends after the window
    s = bench.PowerSampler.summary(rows, 10.0, 14.0)
    assert s["readings"] == 2
    assert s["power_w"] == 1360.0
    assert s["gfx_mhz"] == 1840.0 and s["gfx_mhz_min"] == 1820.0 and s["gfx_mhz_max"] == 1860.0
    assert bench.PowerSampler.summary(rows, 20.0, 30.0) is None


def test_profiler_detection(monkeypatch):
    for k in [k for k in os.environ if k.startswith(("ROCPROF", "ROCP_"))]:
        monkeypatch.delenv(k)
    monkeypatch.setenv("LD_PRELOAD", "")
    assert not bench.under_profiler()
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    assert bench.under_profiler()
