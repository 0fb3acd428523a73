"""Throughput of one TMP shard's fwd + fine-grained-recompute + bwd step on one GPU.

A step is one pass of the whole hot path over one micro-batch of seeded
synthetic input: forward of every block for both sub-batches with the
AllReduce-point sums overlapping the other sub-batch's compute, then the
fine-grained recompute and backward of every block (Oases overlapped
schedule).  By default the overlap is realised with one stream per
sub-batch (each sub-batch's compute and AllReduce points on its own stream,
so one sub-batch's sums run beside the other's compute), issued eagerly.

Prints one JSON line.  ``value`` is the counted (algorithmic) TFLOP/s of the
step at the median per-step time (HIP events on the compute stream).  As
many steps again follow in which every kernel-class launch carries a HIP
event pair in its own dispatch packets: the per-class durations, the
roofline entry (the class with the most time per step) and the fraction of
the AllReduce-point sums' time that ran beside compute kernels come from
those.  Each class is also timed alone in a few serial-schedule steps.  The
CPU baseline is the float64 oracle on this host's cores.
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
DEFAULT_WORKLOAD = "c5_pair_h8192"
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


# Algorithmic work of one launch of each kernel class (averaged over the
# class's launches in a step).  A class is what the executor brackets with one
# pair of HIP events: one GEMM, one attention forward, one attention backward
# (dQ-with-delta + dK/dV kernels), one AllReduce-point sum, one bias column sum
# (float32 only: in bf16 the dW_in GEMM sums its A operand's columns).
KERNEL_CLASSES = ("gemm_fwd", "gemm_dx", "gemm_dw", "attn_fwd", "attn_bwd", "sum", "colsum")


def class_launches(cfg, kclass):
    """Launches of a kernel class in one overlapped fine-grained step."""
    L = cfg.n_layers
    n_attn = sum(1 for b in cfg.blocks if b == gen.ATTN)
    return {"gemm_fwd": 6 * L, "gemm_dx": 4 * L, "gemm_dw": 4 * L, "attn_fwd": 4 * n_attn, "attn_bwd": 2 * n_attn,
            "sum": 4 * L, "colsum": 2 * L}[kclass]


def class_work(cfg, kclass):
    """(algorithmic work of one step for the class, unit): FLOPs or HBM bytes."""
    T, h = cfg.t_sb, cfg.hidden
    esz = 2 if cfg.dtype == gen.BF16 else 4
    tot = 0.0
    for l, kind in enumerate(cfg.blocks):
        nin, nmid = cfg.n_in(l), cfg.n_mid(l)
        col, row = gemm_flops(T, nin, h), gemm_flops(T, h, nmid)
        att = attn_matmul_flops(cfg) if kind == gen.ATTN else 0.0
        if kclass == "gemm_fwd":     # F: column + row, R: column
            tot += 2 * (2 * col + row)
        elif kclass in ("gemm_dx", "gemm_dw"):
            tot += 2 * (col + row)
        elif kclass == "attn_fwd":   # F and R: QK^T and PV
            tot += 2 * 2 * 2 * att
        elif kclass == "attn_bwd":   # dV, dP, dQ, dK
            tot += 2 * 4 * att
        elif kclass == "sum":
            tot += 2 * 2 * (cfg.tmp_width + 1) * T * h * esz
        elif kclass == "colsum" and cfg.dtype != gen.BF16:  # bf16: inside the dW_in GEMM
            tot += 2 * (T * nin * esz + 2 * nin * 4)         # read dpre once, db read-modify-write
    return tot, ("B" if kclass in ("sum", "colsum") else "FLOP")


# ---------------------------------------------------------------------------

def cpu_baseline(cfg, budget_s=12.0, budget_f32_s=4.0):
    """The float64 oracle step on this host (a bounded number of whole steps),
    and the same oracle run in float32 (reported beside it)."""
    import numpy as np
    from oracle import schedule
    inp = gen.make_inputs(cfg)
    flops = sum(step_flops(cfg))

    def timed(dtype, budget):
        t0 = time.perf_counter()
        n = 0
        while True:
            schedule.run_step(inp, "serial_fine", work_dtype=dtype)
            n += 1
            if time.perf_counter() - t0 >= budget or n >= 200:
                return n, (time.perf_counter() - t0) / n

    n, dt = timed(np.float64, budget_s)
    n32, dt32 = timed(np.float32, budget_f32_s)
    cores = len(os.sched_getaffinity(0))
    blas = os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or "default"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} whole fp64 oracle steps of the {cfg.name} workload "
                      f"(serial fine-grained schedule), {dt:.2f} s per step, numpy/OpenBLAS "
                      f"on {cores} cores (BLAS threads: {blas})",
            "fp32_value": flops / dt32 / 1e12,
            "fp32_sample": f"{n32} whole oracle steps in float32, {dt32:.2f} s per step"}


def stored_traffic(kclass, workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) stored
    from two counter runs of this bench, or None when absent or when the
    kernel sources have changed since the counters were taken."""
    from tensor_model_transformer_tmp_amd.rocprof_summary import sources_hash
    path = os.path.join(ROOT, "profiles", f"{kclass}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for ln in fh:
            k, sep, v = ln.partition(":")
            if sep:
                kv[k.strip()] = v.strip()
    if kv.get("sources_sha256") != sources_hash(kclass):
        return None
    return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])


def copy_calibration(nbytes):
    """A plain copy of known size (the sum kernel with no peers), for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    from tensor_model_transformer_tmp_amd import shard
    n = nbytes // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        shard.allreduce_point(shard.BF16, src, src, 0, dst)
    torch.cuda.synchronize()
    assert bool((dst == 1).all())
    print(json.dumps({"copy_bytes": 2 * n, "launches": 3}), flush=True)


# ---------------------------------------------------------------------------
# studies (one JSON line each; not the timed step)
# ---------------------------------------------------------------------------

ABLATION_MODES = ("serial_norecompute", "serial_default", "serial_fine", "overlap_fine",
                  "overlap_fused", "overlap_streams")


def study_ablation(cfg, steps, warmup):
    """Schedule ablation on one GPU with the same kernels (Section IV, Fig. 4;
    the analogue of the pages' schedule comparison table): no recompute
    (every intermediate kept), default recompute (the whole block re-run,
    row GEMM and its AllReduce point included), fine-grained recompute
    serial, and fine-grained recompute overlapped (side stream, or fused into
    the next GEMM launch).  Each mode is timed eagerly and as a hipGraph
    replay; the faster is reported.  ``model_tflops`` divides the model's own
    forward + backward FLOPs (no recompute) by the step time, so the modes are
    compared on equal work; ``executed_tflops`` counts what the mode runs."""
    import torch
    from tensor_model_transformer_tmp_amd.device import DeviceShard

    dev = DeviceShard(gen.make_inputs(cfg), device="cuda:0", modes=ABLATION_MODES)
    f, r, b = step_flops(cfg)
    executed = {"serial_norecompute": f + b, "serial_default": 2 * f + b}
    out = {}
    for mode in ABLATION_MODES:
        best = None
        for graph in (False, True):
            for _ in range(warmup):
                dev.ctx.schedule_step(mode, graph)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                dev.ctx.schedule_step(mode, graph)
            torch.cuda.synchronize()
            t = (time.perf_counter() - t0) / steps
            if best is None or t < best[0]:
                best = (t, graph)
        t, graph = best
        ex = executed.get(mode, f + r + b)
        out[mode] = {"ms_per_step": t * 1e3, "issue": "hipGraph" if graph else "eager",
                     "model_tflops": (f + b) / t / 1e12, "executed_gflop": ex / 1e9,
                     "executed_tflops": ex / t / 1e12}
    dev.close()
    base = out["serial_norecompute"]["ms_per_step"]
    for v in out.values():
        v["speed_vs_norecompute"] = base / v["ms_per_step"]
    return {"study": "schedule_ablation", "workload": cfg.name, "steps": steps,
            "warmup": warmup, "modes": out}


def event_timeline(dev, mode, steps):
    """``steps`` eager steps of ``mode`` with every kernel-class launch timed
    by HIP events carried in its dispatch packets: (figures, text chart) of
    how the launches ran side by side (no profiler attached)."""
    from tensor_model_transformer_tmp_amd.rocprof_summary import overlap_report
    import torch
    cap = 16384
    dev.ctx.profile_begin("all", cap)
    t0 = time.perf_counter()
    for _ in range(steps):
        dev.ctx.schedule_step(mode, False)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    rows = [(a * 1e6, b * 1e6, ("compute", "side", "other")[st], cls, cls)
            for cls, st, a, b in dev.ctx.profile_timeline(cap)]
    fig, text = overlap_report(rows, steps)
    fig["ms_per_step_with_events"] = t * 1e3
    return fig, text


def study_trace(cfg, mode, steps, warmup, timeline_out=None):
    """Steps of one schedule only, issued eagerly, for a kernel trace: warm-up
    and timed steps are all the library runs, so a rocprofv3 kernel trace of
    this command is a timeline of exactly those steps (the trace summary
    measures how much of each AllReduce-point sum ran beside compute
    kernels).  Then the same number of steps again with dispatch-packet
    events on every launch, for the same figures without a profiler."""
    import torch
    from tensor_model_transformer_tmp_amd.device import DeviceShard

    dev = DeviceShard(gen.make_inputs(cfg), device="cuda:0", modes=(mode,))
    for _ in range(warmup):
        dev.ctx.schedule_step(mode, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dev.ctx.schedule_step(mode, False)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    fig, text = event_timeline(dev, mode, steps)
    dev.close()
    if timeline_out:
        with open(timeline_out, "w") as fh:
            fh.write(f"{cfg.name}, {mode} eager, HIP events in every launch's dispatch packets\n"
                     + text + "\n")
    return {"study": "trace", "workload": cfg.name, "schedule": mode + "+eager", "steps": steps,
            "warmup": warmup, "ms_per_step": t * 1e3, "event_timeline": fig}


def power_sampler(out_path, stop_path, max_s=300.0):
    """Child process of --study power (it never touches the GPU through HIP):
    reads the board's socket power and the graphics clocks with amd-smi in a
    loop and appends one JSON line per reading, until the stop file appears."""
    import re
    import subprocess
    t_end = time.time() + max_s
    parent = os.getppid()
    with open(out_path, "a") as fh:
        while not os.path.exists(stop_path) and time.time() < t_end and os.getppid() == parent:
            t = time.time()
            try:
                txt = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                                     timeout=20).stdout
            except (OSError, subprocess.TimeoutExpired):
                fh.write(json.dumps({"t": t, "error": "amd-smi unavailable"}) + "\n")
                return 0
            pw = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", txt)
            clk = [int(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", txt)]
            fh.write(json.dumps({"t": t, "t_done": time.time(), "power_w": float(pw.group(1)) if pw else None,
                                 "gfx_mhz": clk}) + "\n")
            fh.flush()
    return 0


def under_profiler() -> bool:
    """True when running under rocprofv3 (its tool library is preloaded into
    every child process too, so no sampler child may be started then)."""
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return True
    return any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ)


class PowerSampler:
    """amd-smi readings (socket power, per-XCD clock) from a child process,
    started before this process first uses the GPU."""

    def __init__(self, max_s=300.0):
        import subprocess
        import tempfile
        tmp = tempfile.mkdtemp(prefix="oases_power_")
        self.out_path, self.stop_path = os.path.join(tmp, "samples.jsonl"), os.path.join(tmp, "stop")
        self.child = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--power-sampler",
                                       self.out_path, self.stop_path, str(max_s)])

    def stop(self):
        import subprocess
        open(self.stop_path, "w").close()
        try:
            self.child.wait(timeout=60)
        except subprocess.TimeoutExpired:
            self.child.kill()
            self.child.wait()
        rows = []
        if os.path.exists(self.out_path):
            with open(self.out_path) as fh:
                rows = [json.loads(x) for x in fh if x.strip()]
        return rows

    @staticmethod
    def summary(rows, t0, t1):
        """Median power and clock of the readings taken inside [t0 + 1 s, t1]."""
        from statistics import median
        busy = [x for x in rows if x.get("t", 0) >= t0 + 1.0 and x.get("t_done", 1e30) <= t1
                and x.get("power_w") is not None and x.get("gfx_mhz")]
        if not busy:
            return None
        mhz = [sum(x["gfx_mhz"]) / len(x["gfx_mhz"]) for x in busy]
        return {"readings": len(busy), "power_w": median([x["power_w"] for x in busy]),
                "gfx_mhz": median(mhz), "gfx_mhz_min": min(mhz), "gfx_mhz_max": max(mhz)}


def study_power(cfg, mode, seconds, warmup, target="step", tile_variant=0):
    """Board power and graphics clock while the timed step runs (or, with
    target "probe", while the MFMA probe runs back to back: the dense bf16
    rate the chip sustains at its power limit): a child process samples
    amd-smi (socket power, current clock of every XCD) from before the GPU is
    first used until the work ends; readings taken inside the timed window
    (after its first second) are summarised.  The MFMA peak of 2.5 PFLOP/s
    assumes the 2.4 GHz peak clock; the same peak at the measured clock is
    reported beside it."""
    from statistics import median
    if under_profiler():
        return {"study": "power", "note": "not run under a profiler (the sampler child would be profiled too)"}
    sampler = PowerSampler()  # started before this process initialises the GPU
    try:
        import torch
        from tensor_model_transformer_tmp_amd.device import DeviceShard

        time.sleep(2.0)  # idle readings
        t_gpu = time.time()
        from tensor_model_transformer_tmp_amd import shard
        cs = torch.cuda.current_stream()
        if target == "probe":
            wgs = 256 * 4  # 4 workgroups of 4 waves per CU, back-to-back independent MFMAs
            buf = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
            work = lambda: shard.mfma_probe(wgs, 5000, buf)
            flops = work()
            torch.cuda.synchronize()
        elif target == "gemm":
            # the 8192-hidden pair's FFN-out forward GEMM, 2048 x 8192 x 4096, automatic tile
            m_, n_, k_ = 2048, 8192, 4096
            ga = torch.randn(m_, k_, device="cuda:0").to(torch.bfloat16)
            gw = (torch.randn(n_, k_, device="cuda:0") * 0.02).to(torch.bfloat16)
            gc = torch.empty(m_, n_, device="cuda:0", dtype=torch.bfloat16)
            shard.set_gemm_tile_variant(tile_variant)
            work = lambda: shard.gemm(shard.BF16, ga, gw, gc, 0, 0, "store")
            flops = 2.0 * m_ * n_ * k_
        elif target == "sum":
            # one AllReduce point of the 8192-hidden pair: own + 7 peers of 2048 x 8192 bf16
            n_ = 2048 * 8192
            so = torch.ones(n_, dtype=torch.bfloat16, device="cuda:0")
            sp = torch.ones(7, n_, dtype=torch.bfloat16, device="cuda:0")
            sy = torch.empty_like(so)
            work = lambda: shard.allreduce_point(shard.BF16, so, sp, 7, sy)
            flops = 9.0 * n_ * 2  # bytes moved (reported in the TFLOP/s field as TB/s)
        else:
            dev = DeviceShard(gen.make_inputs(cfg), device="cuda:0", modes=(mode,))
            cs = dev.compute
            work = lambda: dev.ctx.schedule_step(mode, False)
            f, r, b = step_flops(cfg)
            flops = f + r + b
        for _ in range(warmup):
            work()
        torch.cuda.synchronize()
        times, t0 = [], time.time()
        while time.time() - t0 < seconds:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cs)
            work()
            e1.record(cs)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        t1 = time.time()
        if target == "step":
            dev.close()
    finally:
        rows = sampler.stop()
    idle = [x for x in rows if x.get("t_done", 0) < t_gpu and x.get("power_w") is not None]
    busy = [x for x in rows if x.get("t", 0) >= t0 + 1.0 and x.get("t_done", 1e30) <= t1
            and x.get("power_w") is not None]
    ms = median(times)
    out = {"study": "power", "target": target, "seconds": seconds, "steps": len(times), "ms_per_step": ms,
           "tflops": flops / (ms / 1e3) / 1e12, "readings_in_window": len(busy)}
    if target == "probe":
        out["workload"] = "mfma_probe (4 workgroups of 4 waves per CU, bf16 32x32x16)"
    elif target == "gemm":
        out["workload"] = "bf16 GEMM 2048 x 8192 x 4096, both operands k-contiguous"
        out["tile_variant"] = tile_variant
    elif target == "sum":
        out["workload"] = "AllReduce-point sum, own + 7 peers of 2048 x 8192 bf16 ('tflops' is TB/s moved)"
    else:
        out.update({"workload": cfg.name, "schedule": mode + "+eager"})
    if target != "step":
        out.pop("ms_per_step")
        out["us_per_launch"] = ms * 1e3
        out["launches"] = out.pop("steps")
    if not busy:
        out["note"] = "no amd-smi readings inside the timed window"
        if rows and "error" in rows[0]:
            out["note"] = rows[0]["error"]
        return out
    mhz = [sum(x["gfx_mhz"]) / len(x["gfx_mhz"]) for x in busy if x["gfx_mhz"]]
    clk = median(mhz)
    out.update({
        "idle_power_w": median([x["power_w"] for x in idle]) if idle else None,
        "power_w": {"median": median([x["power_w"] for x in busy]), "min": min(x["power_w"] for x in busy),
                    "max": max(x["power_w"] for x in busy)},
        "gfx_mhz": {"median": clk, "min": min(mhz), "max": max(mhz)},
        "mfma_bf16_peak_tflops_at_clock": MFMA_BF16_PEAK_TFLOPS * clk / 2400.0,
        "frac_of_peak_at_clock": (None if target == "sum" else
                                  flops / (ms / 1e3) / 1e12 / (MFMA_BF16_PEAK_TFLOPS * clk / 2400.0)),
    })
    return out


def study_peaks(reps=10):
    """The two rooflines measured on this GPU.  MFMA: a probe kernel of
    back-to-back independent bf16 32x32x16 MFMAs with register operands, at
    1, 2 and 4 workgroups of 4 waves per CU.  HBM: torch's device copy, the
    sum kernel with no peers (a copy), and the sum kernel with 3 and 7 peers,
    on buffers well beyond the 256 MB Infinity Cache.  Each is timed with
    events over ``reps`` back-to-back launches; GB/s counts the bytes each
    launch must move."""
    import torch
    from tensor_model_transformer_tmp_amd import shard

    dev = torch.device("cuda:0")
    out = {}
    mfma = {}
    for per_cu in (1, 2, 4):
        wgs = 256 * per_cu
        buf = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
        iters = 20000 // per_cu
        flop = shard.mfma_probe(wgs, iters, buf)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            shard.mfma_probe(wgs, iters, buf)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        mfma[f"{per_cu}_workgroups_per_cu"] = {"flop": flop, "us": sec * 1e6, "TFLOP/s": flop / sec / 1e12}
        del buf

    def timed(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        return {"bytes": nbytes, "us": sec * 1e6, "GB/s": nbytes / sec / 1e9}

    n = 1 << 30  # 1 Gi bf16 elements, 2 GiB per buffer
    a = torch.ones(n, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    out["torch_copy_2GiB"] = timed(lambda: b.copy_(a), 4 * n)
    out["sum_no_peers_2GiB"] = timed(lambda: shard.allreduce_point(shard.BF16, a, a, 0, b), 4 * n)
    del a, b
    # 128 MiB per buffer; then one sub-batch's point of the 8192-hidden pair
    # (2048 x 8192 bf16 = 32 MiB per buffer, 7 peers)
    # both forms of the sum kernel: A (several vectors per thread in flight,
    # the form for sums that run alone) and B (one vector per thread, few
    # registers: the form for sums beside compute)
    for peers, m, name in ((3, 64 << 20, "sum_3_peers_128MiB_each"), (7, 64 << 20, "sum_7_peers_128MiB_each"),
                           (7, 2048 * 8192, "sum_7_peers_2048x8192")):
        own = torch.ones(m, dtype=torch.bfloat16, device=dev)
        pr = torch.ones(peers, m, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(own)
        for form, tag in ((1, ""), (2, "_form_b")):
            shard.set_sum_variant(form)
            out[name + tag] = timed(lambda: shard.allreduce_point(shard.BF16, own, pr, peers, y), (peers + 2) * 2 * m)
        shard.set_sum_variant(0)
        del own, pr, y
    torch.cuda.empty_cache()
    return {"study": "peaks", "reps": reps, "mfma_bf16_peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS, "mfma_probe": mfma,
            "hbm_peak_GB/s": HBM_PEAK_GBS, "hbm": out}


def _gemm_graph_us(shard, torch, M, N, K, reps=20):
    """Average time of one forward-layout GEMM (automatic tiles) over a
    hipGraph of ``reps`` back-to-back launches."""
    dev = torch.device("cuda:0")
    a = torch.randn(M * K, device=dev).to(torch.bfloat16).view(M, K)
    b = torch.randn(N * K, device=dev).to(torch.bfloat16).view(N, K)
    c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
    s = torch.cuda.Stream(device=dev)
    launch = lambda: shard.gemm(shard.BF16, a, b, c, 0, 0, "store", stream=s)
    with torch.cuda.stream(s):
        launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            launch()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def study_kloop():
    """Fixed and per-k cost of a 1024-hidden sub-batch GEMM: 2048 x 1024 x k
    for k = 64 .. 4096, and one 64 x 64 x 64 workgroup, as hipGraph replays;
    the slope over the long-k end is the k loop's incremental rate."""
    import torch
    from tensor_model_transformer_tmp_amd import shard
    ks = (64, 128, 256, 512, 1024, 2048, 4096)
    us = {k: _gemm_graph_us(shard, torch, 2048, 1024, k) for k in ks}
    slope = (us[4096] - us[1024]) / (4096 - 1024)  # us per unit of k
    return {"study": "kloop", "m": 2048, "n": 1024, "us": {str(k): v for k, v in us.items()},
            "one_workgroup_64x64x64_us": _gemm_graph_us(shard, torch, 64, 64, 64),
            "ns_per_k": slope * 1e3, "incremental_tflops": 2 * 2048 * 1024 / (slope * 1e-6) / 1e12}


def _layer_gemms(cfg, l, T):
    """The six GEMMs of block l over T tokens: (name, a_layout, b_layout, M, N, K)."""
    h, nin, nmid = cfg.hidden, cfg.n_in(l), cfg.n_mid(l)
    return [("col_fwd", 0, 0, T, nin, h), ("row_fwd", 0, 0, T, h, nmid),
            ("row_dx", 0, 1, T, nmid, h), ("col_dx", 0, 1, T, h, nin),
            ("row_dw", 1, 1, h, nmid, T), ("col_dw", 1, 1, nin, h, T)]


def study_density(names, reps=20):
    """Batch-split density study (Section IV's argument that splitting a
    micro-batch in two costs little arithmetic density): every GEMM of each
    block at the whole micro-batch (T = B*s tokens) and at one sub-batch
    (T/2), on the same kernels with the automatic tile choice.  Each is timed
    as a hipGraph of ``reps`` back-to-back launches (no host launch cost);
    ``split_loss`` = 1 - t(T) / (2 t(T/2)) summed over the block's GEMMs."""
    import torch
    from tensor_model_transformer_tmp_amd import shard

    dev = torch.device("cuda:0")
    res = []
    for name in names:
        cfg = gen.PRESETS[name]
        kinds = sorted(set(cfg.blocks), key=cfg.blocks.index)
        for kind in kinds:
            l = cfg.blocks.index(kind)
            row = {"workload": name, "block": "attn" if kind == gen.ATTN else "ffn", "gemms": {}}
            tot = {}
            for T in (2 * cfg.t_sb, cfg.t_sb):
                tot[T] = 0.0
                for gname, la, lb, M, N, K in _layer_gemms(cfg, l, T):
                    a = torch.randn(K * M, device=dev).to(torch.bfloat16).view(
                        (M, K) if la == 0 else (K, M))
                    b = torch.randn(K * N, device=dev).to(torch.bfloat16).view(
                        (N, K) if lb == 0 else (K, N))
                    c = torch.empty(M, N, device=dev,
                                    dtype=torch.float32 if la == 1 else torch.bfloat16)
                    epi = "f32" if la == 1 else "store"
                    s = torch.cuda.Stream(device=dev)

                    def launch():
                        shard.gemm(shard.BF16, a, b, c, la, lb, epi, m=M, n=N, k=K, stream=s)

                    with torch.cuda.stream(s):
                        launch()
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        for _ in range(reps):
                            launch()
                    g.replay()
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    with torch.cuda.stream(s):
                        e0.record(s)
                        g.replay()
                        e1.record(s)
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) / reps * 1e3
                    del g
                    tot[T] += us
                    row["gemms"].setdefault(gname, {})[f"T{T}"] = {
                        "shape": [M, N, K], "us": us, "tflops": gemm_flops(M, N, K) / us / 1e6}
            T = 2 * cfg.t_sb
            row["us_whole"], row["us_two_halves"] = tot[T], 2 * tot[cfg.t_sb]
            row["split_loss"] = 1.0 - tot[T] / (2 * tot[cfg.t_sb])
            res.append(row)
    return {"study": "batch_split_density", "reps": reps, "blocks": res}


def _graph_us(torch, s, launch, reps=20, trials=3):
    """Best over ``trials`` of the average time of one launch in a hipGraph of
    ``reps`` back-to-back launches on stream ``s``."""
    with torch.cuda.stream(s):
        launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            launch()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / reps * 1e3)
    del g
    return best


def study_libgemm(cfg):
    """Context for the GEMM rooflines: each distinct GEMM shape of the step
    (one sub-batch, automatic tiles, plain store: bf16 C, float32 C for the
    weight gradients) against the vendor library on the same operands and
    layouts (torch's matmul, which calls hipBLASLt; it writes bf16 C in all
    cases), both as hipGraph replays.  The per-step totals weight each shape
    by its launches in one step (the column GEMM runs in F and in R)."""
    import torch
    from tensor_model_transformer_tmp_amd import shard

    dev = torch.device("cuda:0")
    shapes = {}
    for l in range(cfg.n_layers):
        for gname, la, lb, M, N, K in _layer_gemms(cfg, l, cfg.t_sb):
            key = (gname, la, lb, M, N, K)
            shapes[key] = shapes.get(key, 0) + 2 * (2 if gname == "col_fwd" else 1)  # two sub-batches
    rows, tot_ours, tot_lib = [], 0.0, 0.0
    for (gname, la, lb, M, N, K), launches in shapes.items():
        a = torch.randn(K * M, device=dev).to(torch.bfloat16).view((M, K) if la == 0 else (K, M))
        b = (torch.randn(K * N, device=dev) * 0.05).to(torch.bfloat16).view((N, K) if lb == 0 else (K, N))
        c = torch.empty(M, N, device=dev, dtype=torch.float32 if la == 1 else torch.bfloat16)
        epi = "f32" if la == 1 else "store"
        s = torch.cuda.Stream(device=dev)
        ours = _graph_us(torch, s, lambda: shard.gemm(shard.BF16, a, b, c, la, lb, epi, m=M, n=N, k=K, stream=s))
        ref = c.float().clone()
        if la == 0 and lb == 0:
            lib = lambda: torch.nn.functional.linear(a, b)
        elif la == 0:
            lib = lambda: torch.mm(a, b)
        else:
            at = a.t()
            lib = lambda: torch.mm(at, b)
        lib_us = _graph_us(torch, s, lib)
        with torch.cuda.stream(s):
            r = lib().float()
        torch.cuda.synchronize()
        diff = ((r - ref).abs().max() / r.abs().max()).item()
        f = gemm_flops(M, N, K)
        rows.append({"gemm": gname, "shape": [M, N, K], "layouts": [la, lb], "launches_per_step": launches,
                     "ours_us": ours, "ours_tflops": f / ours / 1e6, "lib_us": lib_us,
                     "lib_tflops": f / lib_us / 1e6, "ours_over_lib_time": ours / lib_us,
                     "max_rel_diff": diff})
        tot_ours += launches * ours
        tot_lib += launches * lib_us
        del a, b, c, ref, r
    return {"study": "libgemm", "workload": cfg.name, "gemms": rows, "step_gemm_us_ours": tot_ours,
            "step_gemm_us_lib": tot_lib, "ours_over_lib_time": tot_ours / tot_lib}


def _preset(name):
    return gen.PRESETS[name] if name in gen.PRESETS else gen.FULL_PRESETS[name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD, choices=gen.PRESET_ORDER + list(gen.FULL_PRESETS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-kernel", default=None, choices=list(KERNEL_CLASSES),
                    help="kernel class for the roofline entry (default: most time per step)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES three times (counter calibration)")
    ap.add_argument("--study", choices=("ablation", "density", "trace", "peaks", "kloop", "libgemm", "power"),
                    default=None,
                    help="run a study instead of the timed step: schedule ablation on --config, "
                         "the batch-split GEMM density study over the bf16 workloads, or "
                         "--steps eager steps of --schedule alone (for a kernel trace), or the "
                         "measured MFMA and HBM rooflines (MFMA probe; copies and sums beyond the "
                         "Infinity Cache), or the fixed and per-k cost of a 1024-hidden GEMM, or "
                         "the step's GEMM shapes of --config against the vendor library, or the "
                         "board power and graphics clock (amd-smi) while --schedule steps run for "
                         "--seconds")
    ap.add_argument("--seconds", type=float, default=5.0, help="--study power: length of the timed window")
    ap.add_argument("--tile-variant", type=int, default=0,
                    help="--study power --power-target gemm: GEMM tile variant (0: automatic)")
    ap.add_argument("--power-target", default="step", choices=("step", "probe", "gemm", "sum"),
                    help="--study power: run the timed step, or back to back the MFMA probe, the "
                         "8192-hidden FFN-out GEMM or one of its AllReduce points")
    ap.add_argument("--power-sampler", nargs="+", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the power and clock readings (amd-smi) after the timed steps")
    ap.add_argument("--schedule", default="overlap_streams",
                    choices=("overlap_streams", "overlap_fine", "overlap_fused", "serial_fine"),
                    help="schedule of the timed steps and of --study trace (default: one stream per "
                         "sub-batch, the fastest realisation of the overlapped schedule)")
    ap.add_argument("--issue", default="eager", choices=("eager", "graph"),
                    help="issue the timed steps eagerly or as hipGraph replays")
    ap.add_argument("--timeline-out", default=None, metavar="PATH",
                    help="--study trace: write the event timeline's text chart here")
    args = ap.parse_args()
    if args.power_sampler:
        a_ = args.power_sampler
        return power_sampler(a_[0], a_[1], float(a_[2]) if len(a_) > 2 else 300.0)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.gpus != 1:
        print(f"bench.py runs one GPU's TMP shard; --gpus {args.gpus} is not supported "
              "(the AllReduce points are emulated with resident peer buffers on one GPU)",
              file=sys.stderr)
        sys.exit(2)

    if args.study == "ablation":
        print(json.dumps(study_ablation(_preset(args.config), args.steps, args.warmup)), flush=True)
        return 0
    if args.study == "trace":
        print(json.dumps(study_trace(_preset(args.config), args.schedule, args.steps, args.warmup,
                                     args.timeline_out)), flush=True)
        return 0
    if args.study == "power":
        print(json.dumps(study_power(_preset(args.config), args.schedule, args.seconds, args.warmup,
                                     args.power_target, args.tile_variant)), flush=True)
        return 0
    if args.study == "kloop":
        print(json.dumps(study_kloop()), flush=True)
        return 0
    if args.study == "libgemm":
        print(json.dumps(study_libgemm(_preset(args.config))), flush=True)
        return 0
    if args.study == "peaks":
        print(json.dumps(study_peaks()), flush=True)
        return 0
    if args.study == "density":
        names = [n for n in gen.PRESET_ORDER if gen.PRESETS[n].dtype == gen.BF16]
        print(json.dumps(study_density(names)), flush=True)
        return 0

    # board power and clock while the timed schedule runs (after the timed
    # region, in a window of its own): the sampler starts before the GPU is used
    sampler = None
    if not (args.no_clock or under_profiler()):
        try:
            sampler = PowerSampler(max_s=600.0)
        except OSError:  # no temporary directory or no interpreter to start: no readings
            sampler = None

    import torch
    from tensor_model_transformer_tmp_amd.device import DeviceShard
    from tensor_model_transformer_tmp_amd.rocprof_summary import overlap_report

    cfg = _preset(args.config)
    inp = gen.make_inputs(cfg)
    mode = args.schedule
    dev = DeviceShard(inp, device="cuda:0", modes=(mode, "serial_fine"))
    del inp
    use_graph = args.issue == "graph"
    cs = dev.compute

    def steps_with_events(n, graph, mode=mode):
        """n steps, each bracketed by HIP events on the compute stream (the
        step forks the side stream from it and joins it back), with a
        synchronize on both sides of the whole run: (wall s, [ms per step])."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(cs)
        for i in range(n):
            dev.ctx.schedule_step(mode, graph)
            ev[i + 1].record(cs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]

    def median(v):
        v = sorted(v)
        return 0.5 * (v[(len(v) - 1) // 2] + v[len(v) // 2])

    for _ in range(args.warmup):
        dev.ctx.schedule_step(mode, use_graph)
    torch.cuda.synchronize()

    # The timed region: the steps alone, each bracketed by events on the
    # compute stream.  Then the same number of eager steps of the same
    # schedule in which every kernel-class launch also carries a HIP event
    # pair in its own dispatch packets (on the stream it is launched on): the
    # per-class durations and the overlap timeline come from those.  The
    # events cost little beside 50-300 us kernels (the 8192-hidden pair) but
    # dominate 5-20 us ones (the 1024-hidden pair): their step time is
    # reported, and the timeline figures are withheld where it exceeds the
    # timed steps' by more than 15%.
    # the instrumented block records at most 65536 launches: long runs
    # instrument their first n_inst steps
    per_step_launches = sum(class_launches(cfg, kc) for kc in KERNEL_CLASSES)
    n_inst = min(args.steps, ((1 << 16) - 64) // per_step_launches)
    cap = per_step_launches * n_inst + 64
    wall, per_step = steps_with_events(args.steps, use_graph)
    dev.ctx.profile_begin("all", cap)
    _, instrumented = steps_with_events(n_inst, False)
    tl = dev.ctx.profile_timeline(cap)
    # each kernel class alone: a few steps of the serial schedule (same
    # kernels, one stream, nothing running beside a launch), events as above
    n_solo = 5
    dev.ctx.profile_begin("all", cap)
    steps_with_events(n_solo, False, "serial_fine")
    tl_solo = dev.ctx.profile_timeline(cap)
    clock = None
    if sampler is not None:
        # 4 s of the timed schedule; amd-smi readings inside it (after its first second)
        tc0 = time.time()
        while time.time() - tc0 < 4.0:
            for _ in range(10):
                dev.ctx.schedule_step(mode, use_graph)
            torch.cuda.synchronize()
        tc1 = time.time()
        clock = PowerSampler.summary(sampler.stop(), tc0, tc1)
    dev.close()

    # (start ns, end ns, stream, class, name)
    rows = [(a * 1e6, b * 1e6, ("compute", "side", "other")[st], cls, cls) for cls, st, a, b in tl]
    solo = {}
    for cls, _, a, b in tl_solo:
        solo.setdefault(cls, []).append((b - a) * 1e3)  # us
    fig, _ = overlap_report(rows, n_inst)
    ms_step = median(per_step)
    trusted = median(instrumented) <= 1.15 * ms_step
    f, r, b = step_flops(cfg)
    flops = f + r + b
    value = flops / (ms_step / 1e3) / 1e12

    n_steps = n_inst
    kernels = {}
    for kc in KERNEL_CLASSES:
        work, unit = class_work(cfg, kc)
        durs = [(b_ - a_) / 1e3 for a_, b_, _, c_, _ in rows if c_ == kc]  # us
        if work == 0 or not durs:
            continue
        per_step_n = len(durs) // n_steps
        assert per_step_n == class_launches(cfg, kc), (kc, len(durs), n_steps)
        avg = sum(durs) / len(durs) / 1e6  # s
        solo_avg = sum(solo[kc]) / len(solo[kc]) / 1e6
        if unit == "FLOP":
            pk, scale, u = (MFMA_BF16_PEAK_TFLOPS if cfg.dtype == gen.BF16 else FP32_PEAK_TFLOPS), 1e12, "TFLOP/s"
        else:
            pk, scale, u = HBM_PEAK_GBS, 1e9, "GB/s"
        wpl = work / per_step_n
        kernels[kc] = {"launches_per_step": per_step_n, "avg_us": avg * 1e6,
                       "median_us": median(durs), "us_per_step": sum(durs) / n_steps,
                       "achieved": wpl / avg / scale, "unit": u, "frac": wpl / avg / scale / pk,
                       "work_per_launch": wpl, "work_unit": unit,
                       "solo_avg_us": solo_avg * 1e6, "solo_achieved": wpl / solo_avg / scale,
                       "solo_frac": wpl / solo_avg / scale / pk}

    k = args.roofline_kernel or max(kernels, key=lambda c: kernels[c]["us_per_step"])
    kk = kernels[k]
    hbm = kk["unit"] == "GB/s"
    roof = {"bound": "hbm" if hbm else "mfma", "achieved": kk["achieved"],
            "peak": HBM_PEAK_GBS if hbm else (MFMA_BF16_PEAK_TFLOPS if cfg.dtype == gen.BF16
                                              else FP32_PEAK_TFLOPS),
            "unit": kk["unit"], "frac": kk["frac"], "traffic": stored_traffic(k, cfg.name),
            "kernel": f"{k}: {kk['launches_per_step'] * n_steps} launches in {n_steps} steps of the timed "
                      f"schedule ({mode}, eager, events in the dispatch packets), avg {kk['avg_us']:.2f} us, "
                      f"{kk['work_per_launch']:.4g} {kk['work_unit']} per launch",
            # the same class alone (serial schedule, after the timed steps): in
            # the timed steps a launch shares the GPU with the other sub-batch's
            # kernels, so its duration is longer than the kernel's own
            "solo": {"achieved": kk["solo_achieved"], "frac": kk["solo_frac"], "avg_us": kk["solo_avg_us"],
                     "launches": kk["launches_per_step"] * n_solo}}

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == gen.BF16 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "blocks": ["attn" if x == gen.ATTN else "ffn"
                                                     for x in cfg.blocks],
                   "micro_batch": cfg.micro_batch, "seq_len": cfg.seq, "hidden": cfg.hidden,
                   "heads_per_shard": cfg.heads_per_shard, "head_dim": cfg.head_dim,
                   "ffn_shard": cfg.ffn_shard, "tmp_width": cfg.tmp_width,
                   "schedule": mode + "+" + ("hipGraph" if use_graph else "eager"),
                   "parallelism": "one TMP shard, 1 GPU",
                   **({"full_block": True, "dropout_p": cfg.drop_q / 65536.0, "gelu_tanh": cfg.gelu_tanh}
                      if cfg.full_block else {})},
        "timing": "median of per-step HIP-event times on the compute stream over the timed steps",
        "wall_ms_per_step": wall / args.steps * 1e3,
        "instrumented_ms_per_step": median(instrumented), "instrumented_steps": n_inst,
        "instrumented_over_timed": median(instrumented) / ms_step,
        "mfma_peak_frac": value / (MFMA_BF16_PEAK_TFLOPS if cfg.dtype == gen.BF16 else FP32_PEAK_TFLOPS),
        # the part of the AllReduce-point sums' time during which a GEMM or
        # attention kernel of either stream was running, over the
        # instrumented steps (null where the events distort the schedule)
        "reduction_hidden_frac": fig["hidden_frac"] if trusted else None,
        "overlap": fig,
        "kernels": kernels,
        "gflop_per_step": {"fwd": f / 1e9, "recompute": r / 1e9, "bwd": b / 1e9},
        "roofline": roof,
        # board power and graphics clock (amd-smi) during 4 s of the timed
        # schedule run after the timed region; the MFMA peak above assumes
        # the 2.4 GHz peak clock
        "clock": (None if clock is None else
                  {**clock, "mfma_bf16_peak_tflops_at_clock": MFMA_BF16_PEAK_TFLOPS * clock["gfx_mhz"] / 2400.0,
                   "value_frac_of_peak_at_clock": value / (MFMA_BF16_PEAK_TFLOPS * clock["gfx_mhz"] / 2400.0)}),
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(cfg),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
