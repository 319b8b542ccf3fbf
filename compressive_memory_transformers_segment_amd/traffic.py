"""HBM traffic per kernel launch from rocprofv3 counter runs.

    python -m compressive_memory_transformers_segment_amd.traffic \\
        --fetch FETCH_DIR --write WRITE_DIR --workload NAME --mode delta \\
        --copy-bytes 1073741824 --command "<the profiled command>"
    python -m compressive_memory_transformers_segment_amd.traffic --trace TRACE_DIR \\
        --workload NAME --mode delta --command "<the profiled command>"

Each directory holds the ``*counter_collection.csv`` of one ``rocprofv3 --pmc``
run (``FETCH_SIZE`` in one, ``WRITE_SIZE`` in the other; the counters read KiB
per dispatch); in ``--command`` (the arguments after ``rocprofv3 --pmc NAME``)
the word COUNTER stands for the counter's name. The same run also copies ``--copy-bytes`` bytes with a plain
device-to-device copy kernel: the factor that maps its counted bytes onto the
bytes it actually moved calibrates the counters of every other kernel.

The summary records, per kernel of the forward pass, the calibrated bytes
fetched and written per launch, and the SHA-256 (first 16 hex digits) of the
sources the kernel is built from. ``load`` returns the figures only while
those sources are unchanged, so a stale count is never reported.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# Kernel name pattern -> sources it is built from (besides the shared headers).
KERNEL_SOURCES = [
    (r"chain_pack_kernel", ["segment_scan_mfma.hip"]),
    (r"fused_bf16_kernel", ["fused_bf16.hip"]),
    (r"fused_f32_kernel", ["fused_f32.hip"]),
    (r"segment_scan_kernel", ["segment_scan.hip"]),
    (r"(gh_kernel|seq_kernel|zsum_kernel|zprefix_kernel)", ["segment_scan_mfma.hip"]),
]
SHARED = ["common.h", "launch.h"]
COPY_KERNEL = "copyBuffer"


def _sources_for(kernel: str):
    for pat, files in KERNEL_SOURCES:
        if re.search(pat, kernel):
            return files + SHARED
    return None


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """Kernel name without the namespace and argument list."""
    k = kernel.replace("(anonymous namespace)::", "")
    k = re.sub(r"^void ", "", k).split("(")[0]
    return k.replace("ia::", "").strip()


def read_counter(directory: str, counter: str) -> Dict[str, list]:
    """Counter values (KiB) per dispatch, grouped by kernel name."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    per: Dict[str, Dict[str, float]] = {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = short_name(row["Kernel_Name"])
                disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                per.setdefault(name, {})
                # a counter may be reported per dimension; sum them per dispatch
                per[name][disp] = per[name].get(disp, 0.0) + float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def summarize(fetch_dir: str, write_dir: str, copy_bytes: int, workload: str, mode: str,
              command: str) -> str:
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if COPY_KERNEL in k]
    copy_w = [v for k, v in write.items() if COPY_KERNEL in k]
    if not copy_f or not copy_w:
        raise RuntimeError("the calibration copy kernel is missing from the counter runs")
    kib = copy_bytes / 1024.0
    # the copy kernel may be split into several dispatches; take the largest
    cf = max(max(v) for v in copy_f)
    cw = max(max(v) for v in copy_w)
    fscale, wscale = kib / cf, kib / cw
    lines = [
        f"# HBM traffic per launch, workload {workload}, {mode} rule",
        "# Commands (repository root, one MI355X, rocprofv3, TMPDIR=/tmp), one counter per run:",
        f"#   rocprofv3 --pmc FETCH_SIZE {command.replace('COUNTER', 'FETCH_SIZE')}",
        f"#   rocprofv3 --pmc WRITE_SIZE {command.replace('COUNTER', 'WRITE_SIZE')}",
        f"# Calibration: a {copy_bytes} byte device-to-device copy reads FETCH_SIZE {cf:.1f} KiB"
        f" and WRITE_SIZE {cw:.1f} KiB;",
        f"# FETCH_SIZE is scaled by {fscale:.4f} and WRITE_SIZE by {wscale:.4f}.",
        "# Per kernel: median KiB per dispatch (dispatches), calibrated bytes per launch.",
        f"workload = {workload}",
        f"mode = {mode}",
        f"fetch_scale = {fscale:.6f}",
        f"write_scale = {wscale:.6f}",
    ]
    for name in sorted(set(fetch) & set(write)):
        if COPY_KERNEL in name:
            continue
        srcs = _sources_for(name)
        if srcs is None:
            continue
        f_kib = statistics.median(fetch[name])
        w_kib = statistics.median(write[name])
        lines.append(f"# {name}: FETCH_SIZE {f_kib:.1f} KiB ({len(fetch[name])}), "
                     f"WRITE_SIZE {w_kib:.1f} KiB ({len(write[name])})")
        lines.append(f"kernel {name} | fetch_bytes = {f_kib * 1024 * fscale:.0f} | "
                     f"write_bytes = {w_kib * 1024 * wscale:.0f} | source_sha256_16 = "
                     f"{source_hash(srcs)}")
    return "\n".join(lines) + "\n"


def path_for(workload: str, mode: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}_{mode}.txt")


def load(workload: str, mode: str) -> Optional[Dict[str, Dict[str, float]]]:
    """Calibrated bytes per launch per kernel, or None when no summary exists
    or any kernel's sources changed since its counters were taken."""
    p = path_for(workload, mode)
    if not os.path.exists(p):
        return None
    out: Dict[str, Dict[str, float]] = {}
    for line in open(p):
        if not line.startswith("kernel "):
            continue
        parts = [x.strip() for x in line[len("kernel "):].split("|")]
        name = parts[0]
        kv = dict(x.split(" = ", 1) for x in parts[1:])
        srcs = _sources_for(name)
        if srcs is None or source_hash(srcs) != kv["source_sha256_16"]:
            return None
        out[name] = {"fetch": float(kv["fetch_bytes"]), "write": float(kv["write_bytes"])}
    return out or None


def trace_table(directory: str, workload: str, mode: str, command: str) -> str:
    """Markdown table of the library's kernels from a ``rocprofv3 --kernel-trace
    --stats`` run (its ``*kernel_stats.csv``), longest first."""
    files = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_stats.csv under {directory}")
    rows = []
    with open(files[0], newline="") as fh:
        for r in csv.DictReader(fh):
            name = short_name(r["Name"])
            if _sources_for(name) is None:
                continue
            rows.append((float(r["TotalDurationNs"]), name, int(r["Calls"]),
                         float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    rows.sort(reverse=True)
    out = [f"# Kernel trace: workload {workload}, {mode} rule", "",
           "Command (repository root, one MI355X, `rocprofv3`, `TMPDIR=/tmp`):", "", "```",
           f"rocprofv3 --kernel-trace --stats {command}", "```", "",
           "Library kernels from `kernel_stats.csv` (warm-up and timed calls; torch's own "
           "kernels left out). The tracer slows the kernels down; bench lines are timed "
           "without it.", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for _, name, calls, avg, mn, mx in rows:
        out.append(f"| `{name}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=int)
    ap.add_argument("--trace", help="format a --kernel-trace --stats run instead")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--mode", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", default=None, help="default: profiles/traffic_<workload>_<mode>.txt "
                                                 "(profiles/kernels_<workload>_<mode>.md with --trace)")
    a = ap.parse_args(argv)
    if a.trace:
        text = trace_table(a.trace, a.workload, a.mode, a.command)
        dst = a.out or os.path.join(PROFILES, f"kernels_{a.workload}_{a.mode}.md")
        with open(dst, "w") as fh:
            fh.write(text)
        sys.stdout.write(text)
        return 0
    if not (a.fetch and a.write and a.copy_bytes):
        ap.error("--fetch, --write and --copy-bytes are required")
    text = summarize(a.fetch, a.write, a.copy_bytes, a.workload, a.mode, a.command)
    dst = a.out or path_for(a.workload, a.mode)
    with open(dst, "w") as fh:
        fh.write(text)
    sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
