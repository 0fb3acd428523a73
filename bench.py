"""Throughput of one TMP shard's fwd + fine-grained-recompute + bwd step on one GPU.

A step is one pass of the whole hot path over one micro-batch of seeded
synthetic input: forward of every block for both sub-batches with the
AllReduce-point sums on the side stream, then the fine-grained recompute and
backward of every block (Oases overlapped schedule), replayed as one hipGraph.

Prints one JSON line.  ``value`` is the counted (algorithmic) TFLOP/s of the
step; the roofline entry is for the dominant kernel, timed with HIP events on
its own stream; the CPU baseline is the float64 oracle on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gen  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 vector
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "c2_pair_h1024"
METRIC = "TMP-shard fwd+recompute+bwd TFLOP/s per GPU; % MFMA peak; % reduction hidden"


# ---------------------------------------------------------------------------
# counted work (algorithmic: causal attention counts the lower triangle only,
# the recompute skips the dead row-parallel GEMM)
# ---------------------------------------------------------------------------

def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def attn_matmul_flops(cfg):
    """One attention matmul (QK^T or PV) over a sub-batch, causal lower triangle."""
    s, d = cfg.seq, cfg.head_dim
    pairs = s * (s + 1) / 2 if cfg.causal else s * s
    return 2.0 * (cfg.micro_batch // 2) * cfg.heads_per_shard * pairs * d


def step_flops(cfg):
    """(forward, recompute, backward) counted FLOPs of one step (both sub-batches)."""
    T, h = cfg.t_sb, cfg.hidden
    f = r = b = 0.0
    for l, kind in enumerate(cfg.blocks):
        nin, nmid = cfg.n_in(l), cfg.n_mid(l)
        col, row = gemm_flops(T, nin, h), gemm_flops(T, h, nmid)
        att = 2 * attn_matmul_flops(cfg) if kind == gen.ATTN else 0.0
        f += col + att + row
        r += col + att
        b += 2 * col + 2 * row + (4 * attn_matmul_flops(cfg) if kind == gen.ATTN else 0.0)
    return 2 * f, 2 * r, 2 * b


def sum_bytes(cfg):
    """HBM bytes of all AllReduce-point sums of a step: (w+1) T h elements per point."""
    esz = 2 if cfg.dtype == gen.BF16 else 4
    return 2 * 2 * cfg.n_layers * (cfg.tmp_width + 1) * cfg.t_sb * cfg.hidden * esz


# flops of one launch of each GEMM kind (for the dominant-kernel roofline)
def gemm_class_flops(cfg, kclass):
    T, h = cfg.t_sb, cfg.hidden
    tot = 0.0
    for l, kind in enumerate(cfg.blocks):
        nin, nmid = cfg.n_in(l), cfg.n_mid(l)
        if kclass == "gemm_fwd":   # F: column + row, R: column (per sub-batch)
            tot += 2 * (2 * gemm_flops(T, nin, h) + gemm_flops(T, h, nmid))
        elif kclass in ("gemm_dx", "gemm_dw"):
            tot += 2 * (gemm_flops(T, nin, h) + gemm_flops(T, h, nmid))
    return tot


def gemm_class_launches(cfg, kclass):
    L = cfg.n_layers
    return {"gemm_fwd": 6 * L, "gemm_dx": 4 * L, "gemm_dw": 4 * L}[kclass]


# ---------------------------------------------------------------------------

def cpu_baseline(cfg, budget_s=12.0):
    """The float64 oracle step on this host (a bounded number of whole steps)."""
    from oracle import schedule
    inp = gen.make_inputs(cfg)
    flops = sum(step_flops(cfg))
    t0 = time.perf_counter()
    n = 0
    while True:
        schedule.run_step(inp, "serial_fine")
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= 20:
            break
    dt = (time.perf_counter() - t0) / n
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} whole fp64 oracle steps of the {cfg.name} workload "
                      f"(serial fine-grained schedule), {dt:.2f} s per step, numpy/OpenBLAS "
                      f"on {cores} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD, choices=gen.PRESET_ORDER)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-kernel", default="gemm_fwd",
                    choices=["gemm_fwd", "gemm_dx", "gemm_dw", "sum"])
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs one GPU's TMP shard; --gpus {args.gpus} is not supported "
              "(the AllReduce points are emulated with resident peer buffers on one GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tensor_model_transformer_tmp_amd.device import DeviceShard

    cfg = gen.PRESETS[args.config]
    inp = gen.make_inputs(cfg)
    dev = DeviceShard(inp, device="cuda:0", modes=("overlap_fine", "serial_fine"))
    del inp

    def run(mode, graph, n):
        for _ in range(n):
            dev.ctx.schedule_step(mode, graph)

    def timed(mode, graph, steps, warmup):
        run(mode, graph, warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(mode, graph, steps)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    # The overlapped fine-grained schedule is issued either eagerly on the two
    # streams or as one captured hipGraph per step; both are timed briefly and
    # the faster one is the timed region.  The same kernels serialised on one
    # stream give the reference for the hidden-reduction estimate.
    probe = max(3, args.steps // 5)
    launch = {g: timed("overlap_fine", g, probe, 2) for g in (False, True)}
    use_graph = launch[True] <= launch[False]
    sec = timed("overlap_fine", use_graph, args.steps, args.warmup)
    sec_serial = timed("serial_fine", use_graph, max(5, args.steps // 2), 3)

    # dominant-kernel and sum-kernel timing: eager steps with HIP events on the launch stream
    def class_time(kclass, steps):
        dev.ctx.profile_begin(kclass, 8192)
        run("overlap_fine", False, steps)
        ms, n = dev.ctx.profile_end()
        return ms / 1e3, n

    prof_steps = max(3, min(args.steps, 20))
    k = args.roofline_kernel
    k_sec, k_n = class_time(k, prof_steps)
    sum_sec, sum_n = class_time("sum", prof_steps)
    dev.close()

    f, r, b = step_flops(cfg)
    flops = f + r + b
    value = flops / sec / 1e12
    sum_per_step = sum_sec / prof_steps
    hidden = (sec_serial - sec) / sum_per_step if sum_per_step > 0 else None
    if k == "sum":
        per_launch = sum_bytes(cfg) / (4 * cfg.n_layers)
        achieved = per_launch / (k_sec / k_n) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    else:
        per_launch = gemm_class_flops(cfg, k) / gemm_class_launches(cfg, k)
        achieved = per_launch / (k_sec / k_n) / 1e12
        peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == gen.BF16 else FP32_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["kernel"] = f"{k} ({k_n} launches timed over {prof_steps} eager steps)"

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": sec * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == gen.BF16 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "blocks": ["attn" if x == gen.ATTN else "ffn"
                                                     for x in cfg.blocks],
                   "micro_batch": cfg.micro_batch, "seq_len": cfg.seq, "hidden": cfg.hidden,
                   "heads_per_shard": cfg.heads_per_shard, "head_dim": cfg.head_dim,
                   "ffn_shard": cfg.ffn_shard, "tmp_width": cfg.tmp_width,
                   "schedule": "overlap_fine+" + ("hipGraph" if use_graph else "eager-2-streams"),
                   "parallelism": "one TMP shard, 1 GPU"},
        "mfma_peak_frac": value / MFMA_BF16_PEAK_TFLOPS,
        "reduction_hidden_frac": hidden,
        "serial_ms_per_step": sec_serial * 1e3,
        "launch_probe_ms": {"eager": launch[False] * 1e3, "graph": launch[True] * 1e3},
        "sum_ms_per_step": sum_per_step * 1e3,
        "sum_hbm_gbs": sum_bytes(cfg) / sum_per_step / 1e9 if sum_per_step > 0 else None,
        "gflop_per_step": {"fwd": f / 1e9, "recompute": r / 1e9, "bwd": b / 1e9},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(cfg),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
