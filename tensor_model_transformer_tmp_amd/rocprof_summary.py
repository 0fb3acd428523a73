"""Per-kernel-class summaries of rocprofv3 CSV output for liboases_shard.

The executor times its kernels in classes (one class launch = one pair of HIP
events on the launch stream): ``gemm_fwd`` / ``gemm_dx`` / ``gemm_dw`` (one
GEMM each), ``attn_fwd`` (one kernel), ``attn_bwd`` (dQ with delta, then dK/dV
kernels), ``sum`` (one AllReduce-point sum), ``colsum`` (two passes).  This
module maps rocprofv3 kernel names onto the same classes so that a kernel
trace and a counter run can be set beside the event timings.

  python -m tensor_model_transformer_tmp_amd.rocprof_summary stats  <kernel_stats.csv>
  python -m tensor_model_transformer_tmp_amd.rocprof_summary traffic --kernel K \
      --fetch <counter_collection.csv> --write <counter_collection.csv> \
      --calib-fetch <csv> --calib-write <csv> --calib-bytes N
  python -m tensor_model_transformer_tmp_amd.rocprof_summary traffic-all --workload W \
      --outdir profiles ... (same inputs; one <class>_<W>_traffic.txt per class)

  python -m tensor_model_transformer_tmp_amd.rocprof_summary timeline <kernel_trace.csv> --steps K --warmup W
  python -m tensor_model_transformer_tmp_amd.rocprof_summary mfma <counter_collection.csv> [--workload W]

``timeline`` reads a kernel trace of ``bench.py --study trace`` (W warm-up
steps, then K plain steps of one schedule, then K with events), measures how much of every
AllReduce-point sum ran while a compute kernel (GEMM or attention) was running
on the GPU, and draws one step as a per-queue text chart.  ``mfma`` averages
the MFMA busy fraction (``MfmaUtil``, weighted by each dispatch's active
cycles) and the executed bf16 MFMA FLOPs per class launch.

``traffic`` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the
same counters read for a plain copy of known size (the sum kernel with no
peers), and prints the per-class-launch HBM bytes together with a hash of the
kernel sources, so that a stored figure can be recognised as stale.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import subprocess
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# kernels whose launch count is the class launch count (the other kernels of a
# multi-kernel class add their time to it)
_LEAD = {"attn_bwd": "attn_dkdv", "colsum": "colsum_pass1", "ln_bwd": "ln_bwd"}

SOURCES = {
    "gemm_fwd": ("gemm_bf16.hip", "gemm_f32.hip"),
    "gemm_dx": ("gemm_bf16.hip", "gemm_f32.hip"),
    "gemm_dw": ("gemm_bf16.hip", "gemm_f32.hip"),
    "attn_fwd": ("attention.hip",),
    "attn_bwd": ("attention.hip",),
    "sum": ("elementwise.hip",),
    "colsum": ("elementwise.hip",),
    "ln_fwd": ("elementwise.hip",),
    "ln_bwd": ("elementwise.hip",),
    "dropout_bwd": ("elementwise.hip",),
}


def sources_hash(kclass: str) -> str:
    """sha256 over the sources a kernel class is compiled from."""
    h = hashlib.sha256()
    for f in SOURCES[kclass] + ("common.h", "kernels.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _demangle(names):
    mangled = [n for n in names if n.startswith("_Z")]
    if not mangled:
        return {n: n for n in names}
    try:
        out = subprocess.run(["c++filt"], input="\n".join(mangled), capture_output=True,
                             text=True, check=True).stdout.splitlines()
    except (OSError, subprocess.CalledProcessError):
        out = mangled
    m = dict(zip(mangled, out))
    return {n: m.get(n, n) for n in names}


_GEMM = re.compile(r"gemm_(?:bf16|f32)_kernel<.*?\(oases::Layout\)(\d), \(oases::Layout\)(\d)")


def kernel_class(name: str):
    """Kernel class of a (demangled) kernel name, or None for other kernels."""
    m = _GEMM.search(name)
    if m:
        return {("0", "0"): "gemm_fwd", ("0", "1"): "gemm_dx", ("1", "1"): "gemm_dw"}.get(m.groups())
    for key, cls in (("attn_fwd", "attn_fwd"), ("attn_dkdv", "attn_bwd"), ("attn_dq", "attn_bwd"),
                     ("attn_delta", "attn_bwd"), ("allreduce_", "sum"), ("colsum_pass", "colsum"),
                     ("ln_fwd", "ln_fwd"), ("ln_bwd", "ln_bwd"), ("ln_grad_pass1", "ln_bwd"),
                     ("dropout_bwd_kernel", "dropout_bwd")):
        if key in name:
            return cls
    return None


def _is_lead(name: str, cls: str) -> bool:
    return cls not in _LEAD or _LEAD[cls] in name


def stats_table(path: str) -> str:
    """Per-kernel rows of a rocprofv3 kernel_stats.csv and per-class totals."""
    with open(path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    names = _demangle([r["Name"] for r in rows])
    out = ["kernel | calls | total us | avg us | min us | max us | class",
           "---|---|---|---|---|---|---"]
    agg = defaultdict(lambda: [0, 0.0])
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = names[r["Name"]]
        cls = kernel_class(n)
        calls, tot = int(r["Calls"]), float(r["TotalDurationNs"])
        short = n.replace("(anonymous namespace)::", "").replace("(oases::Layout)", "L").replace("oases::", "")
        short = re.sub(r"^void ", "", re.sub(r"\(.*$", "", short))
        out.append(f"{short[:90]} | {calls} | {tot / 1e3:.1f} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {cls or '-'}")
        if cls:
            agg[cls][1] += tot
            if _is_lead(n, cls):
                agg[cls][0] += calls
    out += ["", "class | class launches | total us | avg us per class launch", "---|---|---|---"]
    for cls, (calls, tot) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append(f"{cls} | {calls} | {tot / 1e3:.1f} | {tot / max(calls, 1) / 1e3:.2f}")
    return "\n".join(out)


def pmc_per_class(path: str, counter: str):
    """{class: (class launches, mean counter value per class launch)} from a
    rocprofv3 counter_collection.csv (one row per dispatch and counter)."""
    with open(path, newline="") as fh:
        rows = [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    names = _demangle(sorted({r["Kernel_Name"] for r in rows}))
    tot, launches = defaultdict(float), defaultdict(int)
    for r in rows:
        n = names[r["Kernel_Name"]]
        cls = kernel_class(n)
        if cls is None:
            continue
        tot[cls] += float(r["Counter_Value"])
        if _is_lead(n, cls):
            launches[cls] += 1
    return {c: (launches[c], tot[c] / max(launches[c], 1)) for c in tot}


def traffic_lines(kernel, fetch_csv, write_csv, cf_csv, cw_csv, calib_bytes):
    fetch = pmc_per_class(fetch_csv, "FETCH_SIZE").get(kernel)
    write = pmc_per_class(write_csv, "WRITE_SIZE").get(kernel)
    if fetch is None or write is None:
        return None
    cf = pmc_per_class(cf_csv, "FETCH_SIZE")["sum"]
    cw = pmc_per_class(cw_csv, "WRITE_SIZE")["sum"]
    kf, kw = calib_bytes / cf[1], calib_bytes / cw[1]
    return [f"copy calibration: {calib_bytes:.0f} B read and written per launch of the sum kernel "
            f"with no peers; FETCH_SIZE {cf[1]:.1f} -> {kf:.2f} B per unit; "
            f"WRITE_SIZE {cw[1]:.1f} -> {kw:.2f} B per unit",
            f"kernel class: {kernel} ({fetch[0]} launches in the FETCH_SIZE run, "
            f"{write[0]} in the WRITE_SIZE run)",
            f"fetch_bytes_per_launch: {fetch[1] * kf:.0f}",
            f"write_bytes_per_launch: {write[1] * kw:.0f}",
            f"sources_sha256: {sources_hash(kernel)}"]


def _trace_rows(path: str):
    """Kernel dispatches of a rocprofv3 kernel_trace.csv as
    (start_ns, end_ns, queue, class or None, short name), sorted by start."""
    with open(path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    names = _demangle(sorted({r["Kernel_Name"] for r in rows}))
    out = []
    for r in rows:
        n = names[r["Kernel_Name"]]
        short = re.sub(r"\(.*$", "", n.replace("(anonymous namespace)::", "").replace("oases::", ""))
        short = re.sub(r"^void ", "", short)
        q = r.get("Queue_Id") or r.get("Stream_Id") or "0"
        out.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), q, kernel_class(n), short))
    out.sort()
    return out


def _union_len(iv):
    """Total length of the union of intervals [(a, b), ...]."""
    tot, cur_a, cur_b = 0, None, None
    for a, b in sorted(iv):
        if cur_b is None or a > cur_b:
            if cur_b is not None:
                tot += cur_b - cur_a
            cur_a, cur_b = a, b
        else:
            cur_b = max(cur_b, b)
    return tot + (cur_b - cur_a if cur_b is not None else 0)


_LETTER = {"gemm_fwd": "F", "gemm_dx": "X", "gemm_dw": "W", "attn_fwd": "a", "attn_bwd": "b",
           "sum": "S", "colsum": "c", "ln_fwd": "n", "ln_bwd": "m", "dropout_bwd": "d"}


def timed_trace_rows(path: str, steps: int, warmup: int, total=None):
    """The classified dispatches of ``steps`` steps after the first ``warmup``
    of a kernel trace whose classified dispatches are ``total`` equal steps
    (every step of one workload issues the same kernels).  ``total`` defaults
    to warmup + 2 steps: ``bench.py --study trace`` runs ``warmup`` steps,
    ``steps`` plain steps and ``steps`` steps with events on every launch, and
    nothing else of the library."""
    rows = [r for r in _trace_rows(path) if r[3] is not None]
    per_step = len(rows) // (total if total else warmup + 2 * steps)
    return rows[warmup * per_step:(warmup + steps) * per_step]


def overlap_report(rows, steps: int, width: int = 120, unit: float = 1e3) -> tuple:
    """(figures, text) for the dispatches of ``steps`` whole steps, given as
    (start, end, queue, class, name) with times in ns (``unit`` = 1e3 per us).

    hidden fraction = the part of the AllReduce-point sums' time during which
    at least one compute kernel (any other class) was running on the GPU."""
    rows = sorted(rows)
    t0, t1 = rows[0][0], max(r[1] for r in rows)
    sums = [r for r in rows if r[3] == "sum"]
    compute = [(r[0], r[1]) for r in rows if r[3] != "sum"]
    tot_sum = sum(r[1] - r[0] for r in sums)
    covered = 0
    for a, b, *_ in sums:
        covered += _union_len([(max(a, c0), min(b, c1)) for c0, c1 in compute if c0 < b and c1 > a])
    busy = _union_len([(r[0], r[1]) for r in rows])
    qs = sorted({r[2] for r in rows})
    per_step = len(rows) // max(steps, 1)
    fig = {"steps": steps, "launches_per_step": per_step, "span_us_per_step": (t1 - t0) / unit / steps,
           "sum_us_per_step": tot_sum / unit / steps, "sum_beside_compute_us_per_step": covered / unit / steps,
           "hidden_frac": covered / tot_sum if tot_sum else None, "busy_frac": busy / (t1 - t0),
           "kernel_time_over_span": sum(r[1] - r[0] for r in rows) / (t1 - t0)}
    out = [f"timed steps: {steps}; timed launches: {len(rows)} ({per_step} per step) on "
           f"{len(qs)} queue(s); span {fig['span_us_per_step']:.1f} us per step",
           f"AllReduce-point sums: {len(sums)} launches, {fig['sum_us_per_step']:.1f} us per step; "
           f"time during which a compute kernel was also running: "
           f"{fig['sum_beside_compute_us_per_step']:.1f} us per step -> hidden fraction "
           f"{fig['hidden_frac'] if fig['hidden_frac'] is not None else float('nan'):.3f}",
           f"GPU busy (any kernel running): {fig['busy_frac']:.3f} of the span; "
           f"sum of kernel durations / span: {fig['kernel_time_over_span']:.2f}",
           ""]
    # one step: the launches of the middle timed step (steps end with a join
    # of the streams, so consecutive steps do not overlap)
    k = steps // 2
    step = rows[k * per_step:(k + 1) * per_step]
    s0 = step[0][0]
    span = max(max(r[1] for r in step) - s0, 1)
    out.append(f"step {k}: {span / unit:.1f} us; one character = {span / width / unit:.2f} us; "
               + ", ".join(f"{v} {c}" for c, v in _LETTER.items()) + ", . idle")
    for q in qs:
        line = ["."] * width
        for a, b, qq, cls, _ in step:
            if qq != q:
                continue
            i0 = int((a - s0) * width / span)
            i1 = max(i0 + 1, int((b - s0) * width / span))
            for i in range(i0, min(i1, width)):
                line[i] = _LETTER.get(cls, "?")
        out.append(f"queue {q!s:>3} |{''.join(line)}|")
    out += ["", "start us | end us | queue | class | kernel", "---|---|---|---|---"]
    for a, b, q, cls, n in step:
        out.append(f"{(a - s0) / unit:.1f} | {(b - s0) / unit:.1f} | {q} | {cls} | {n[:80]}")
    return fig, "\n".join(out)


def timeline(path: str, steps: int, warmup: int, width: int = 120, total=None) -> str:
    """Hidden-sum figures over the timed steps of a kernel trace and a text
    chart of one step."""
    rows = timed_trace_rows(path, steps, warmup, total)
    if not rows:
        return "no classified kernels in the trace"
    return overlap_report(rows, steps, width)[1]


def mfma_table(path: str, work=None) -> str:
    """Per class: MFMA busy fraction (MfmaUtil weighted by GRBM_GUI_ACTIVE) and
    executed bf16 MFMA FLOPs per class launch (MfmaFlopsBF16, or
    SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512).  ``work``: {class: algorithmic FLOPs
    per class launch}, printed beside the executed figure when given."""
    with open(path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    names = _demangle(sorted({r["Kernel_Name"] for r in rows}))
    disp = defaultdict(dict)
    for r in rows:
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
        disp[key][r["Counter_Name"]] = float(r["Counter_Value"])
    util_w, act, flops = (defaultdict(float) for _ in range(3))
    launches = defaultdict(int)
    for (_, kname), c in disp.items():
        n = names[kname]
        cls = kernel_class(n)
        if cls is None:
            continue
        a = c.get("GRBM_GUI_ACTIVE", 1.0)
        if "MfmaUtil" in c:
            util_w[cls] += c["MfmaUtil"] * a
            act[cls] += a
        flops[cls] += c.get("MfmaFlopsBF16", c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512)
        if _is_lead(n, cls):
            launches[cls] += 1
    out = ["class | class launches | MFMA busy % | executed bf16 MFMA GFLOP per launch"
           + (" | algorithmic GFLOP per launch | executed / algorithmic" if work else ""),
           "---|---|---|---" + ("|---|---" if work else "")]
    for cls in sorted(launches, key=lambda c: -flops[c]):
        n = max(launches[cls], 1)
        line = (f"{cls} | {launches[cls]} | {util_w[cls] / act[cls] if act[cls] else float('nan'):.1f} | "
                f"{flops[cls] / n / 1e9:.3f}")
        if work and cls in work and work[cls] > 0:
            line += f" | {work[cls] / 1e9:.3f} | {flops[cls] / n / work[cls]:.3f}"
        elif work:
            line += " | - | -"
        out.append(line)
    return "\n".join(out)


def util_table(path: str) -> str:
    """Per class, every percentage metric of a rocprofv3 counter run (the
    derived ``*Util`` metrics, e.g. LdsUtil = LDS busy cycles for indexed
    accesses over active cycles, MfmaUtil), averaged over the class's
    dispatches weighted by GRBM_GUI_ACTIVE, and every raw SQ_ counter as its
    mean per class launch."""
    with open(path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    names = _demangle(sorted({r["Kernel_Name"] for r in rows}))
    disp = defaultdict(dict)
    for r in rows:
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
        disp[key][r["Counter_Name"]] = float(r["Counter_Value"])
    metrics = sorted({k for c in disp.values() for k in c if k.endswith("Util")})
    raw = sorted({k for c in disp.values() for k in c if k.startswith("SQ_")})
    wsum = defaultdict(lambda: defaultdict(float))
    act = defaultdict(float)
    launches = defaultdict(int)
    for (_, kname), c in disp.items():
        n = names[kname]
        cls = kernel_class(n)
        if cls is None:
            continue
        a = c.get("GRBM_GUI_ACTIVE", 1.0)
        act[cls] += a
        for m in metrics:
            wsum[cls][m] += c.get(m, 0.0) * a
        for m in raw:
            wsum[cls][m] += c.get(m, 0.0)
        if _is_lead(n, cls):
            launches[cls] += 1
    head = ["class", "class launches"] + [f"{m} %" for m in metrics] + [f"{m} per launch" for m in raw]
    out = [" | ".join(head), "|".join(["---"] * len(head))]
    for cls in sorted(launches, key=lambda c: -act[c]):
        vals = [f"{wsum[cls][m] / act[cls]:.1f}" for m in metrics]
        vals += [f"{wsum[cls][m] / max(launches[cls], 1):.4g}" for m in raw]
        out.append(" | ".join([cls, str(launches[cls])] + vals))
    return "\n".join(out)


def _class_work_per_launch(workload: str):
    """Algorithmic FLOPs per class launch of a named workload (bench.py's counts)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    import gen
    cfg = gen.PRESETS[workload] if workload in gen.PRESETS else gen.FULL_PRESETS[workload]
    out = {}
    for kc in bench.KERNEL_CLASSES:
        w, unit = bench.class_work(cfg, kc)
        if unit == "FLOP" and w > 0:
            out[kc] = w / bench.class_launches(cfg, kc)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("timeline")
    t.add_argument("csv")
    t.add_argument("--steps", type=int, required=True)
    t.add_argument("--warmup", type=int, required=True)
    t.add_argument("--width", type=int, default=120)
    t.add_argument("--total-steps", type=int, default=None,
                   help="steps in the whole trace (default: warmup + 2 steps, the --study trace layout)")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--workload", default=None)
    u = sub.add_parser("util")
    u.add_argument("csv")
    for name in ("traffic", "traffic-all"):
        t = sub.add_parser(name)
        if name == "traffic":
            t.add_argument("--kernel", required=True, choices=sorted(SOURCES))
        else:
            t.add_argument("--workload", required=True)
            t.add_argument("--outdir", required=True)
            t.add_argument("--header", default="", help="text placed before the figures")
        t.add_argument("--fetch", required=True)
        t.add_argument("--write", required=True)
        t.add_argument("--calib-fetch", required=True)
        t.add_argument("--calib-write", required=True)
        t.add_argument("--calib-bytes", type=float, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv))
        return 0
    if a.cmd == "timeline":
        print(timeline(a.csv, a.steps, a.warmup, a.width, a.total_steps))
        return 0
    if a.cmd == "util":
        print(util_table(a.csv))
        return 0
    if a.cmd == "mfma":
        print(mfma_table(a.csv, _class_work_per_launch(a.workload) if a.workload else None))
        return 0
    args = (a.fetch, a.write, a.calib_fetch, a.calib_write, a.calib_bytes)
    if a.cmd == "traffic":
        print("\n".join(traffic_lines(a.kernel, *args)))
        return 0
    for kernel in sorted(SOURCES):
        lines = traffic_lines(kernel, *args)
        if lines is None:
            continue
        path = os.path.join(a.outdir, f"{kernel}_{a.workload}_traffic.txt")
        with open(path, "w") as fh:
            fh.write(a.header + "\n".join(lines) + "\n")
        print("wrote", path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
