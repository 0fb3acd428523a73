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
_LEAD = {"attn_bwd": "attn_dkdv", "colsum": "colsum_pass1"}

SOURCES = {
    "gemm_fwd": ("gemm_bf16.hip", "gemm_f32.hip"),
    "gemm_dx": ("gemm_bf16.hip", "gemm_f32.hip"),
    "gemm_dw": ("gemm_bf16.hip", "gemm_f32.hip"),
    "attn_fwd": ("attention.hip",),
    "attn_bwd": ("attention.hip",),
    "sum": ("elementwise.hip",),
    "colsum": ("elementwise.hip",),
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
                     ("attn_delta", "attn_bwd"), ("allreduce_", "sum"), ("colsum_pass", "colsum")):
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
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
