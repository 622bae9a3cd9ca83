"""Summarize rocprofv3 CSV output into short text files.

Two summaries:

``stats``   per-kernel dispatch counts and durations from a
            ``--kernel-trace --stats`` run (``*_kernel_stats.csv``);
``traffic`` HBM bytes per launch of one kernel from two ``--pmc`` runs
            (``FETCH_SIZE``, then ``WRITE_SIZE``; ``*_counter_collection.csv``).
            Each counter is scaled by what it reads for a plain device copy of
            known size in the same run (the benchmark's ``--copy-calibration``:
            three 1 GiB copies by the HIP runtime's copy kernel), so the result
            is in bytes whatever unit or subset of channels the counter covers.

Usage:
  python -m residual_add_rmsnorm_rows_amd.rocprof_summary stats CSV --command CMD --out FILE
  python -m residual_add_rmsnorm_rows_amd.rocprof_summary traffic --fetch CSV --write CSV \\
      --kernel SUBSTR --bench-out FILE --command CMD --out FILE [--entry SECONDARY_NAME]
"""

from __future__ import annotations

import argparse
import csv
import json
import statistics
import sys
from typing import Dict, List

COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _rows(path: str) -> List[Dict[str, str]]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats(csv_path: str, command: str, notes=(), trace_path: str = "") -> str:
    rows = _rows(csv_path)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        "# rocprofv3 --kernel-trace --stats summary",
        f"# command: {command}",
        *[f"# {n}" for n in notes],
        "# columns: calls  avg_us  min_us  max_us  total_ms  kernel",
    ]
    for r in rows:
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} {float(r['MinNs']) / 1e3:10.3f} "
                     f"{float(r['MaxNs']) / 1e3:10.3f} {float(r['TotalDurationNs']) / 1e6:10.3f}  {r['Name']}")
    if trace_path:
        # kernels dispatched with several grid sizes (workloads sharing a
        # compiled kernel): the same figures per grid size, from the trace
        per = {}
        for r in _rows(trace_path):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            per.setdefault(r["Kernel_Name"], {}).setdefault(grid, []).append(dur)
        split = [(name, g, d) for name, grids in per.items() if len(grids) > 1 for g, d in grids.items()]
        if split:
            lines.append("# per grid size (threads), for kernels launched with more than one; from the kernel trace")
            lines.append("# columns: calls  avg_us  min_us  max_us  total_ms  grid  kernel")
            split.sort(key=lambda t: -sum(t[2]))
            for name, g, d in split:
                lines.append(f"{len(d):7d} {statistics.mean(d):10.3f} {min(d):10.3f} {max(d):10.3f} "
                             f"{sum(d) / 1e3:10.3f} {g:>10d}  {name}")
    return "\n".join(lines) + "\n"


def _counter(rows, counter: str, match) -> List[float]:
    return [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and match(r)]


def _copy_rows(rows, counter: str):
    """The calibration copies: the runtime copy kernel's dispatches with the
    largest reading (the 1 GiB copies are the largest copies the benchmark
    makes; its other copies, e.g. tensor clones, share the same grid)."""
    copies = [r for r in rows if r["Kernel_Name"] == COPY_KERNEL and r["Counter_Name"] == counter]
    if not copies:
        raise SystemExit("no copy-calibration dispatches in the counter file")
    top = max(float(r["Counter_Value"]) for r in copies)
    ids = {r["Dispatch_Id"] for r in copies if float(r["Counter_Value"]) >= 0.99 * top}
    return lambda r: r["Kernel_Name"] == COPY_KERNEL and r["Dispatch_Id"] in ids


def _last_json(path: str) -> dict:
    with open(path) as f:
        lines = [l for l in f if l.startswith("{")]
    if not lines:
        raise SystemExit(f"no JSON line in {path}")
    return json.loads(lines[-1])


def traffic(fetch_csv: str, write_csv: str, kernel: str, bench_out: str, command: str, entry: str = "",
            grid_size: int = 0) -> str:
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    names = sorted({r["Kernel_Name"] for r in fr + wr if kernel in r["Kernel_Name"]})
    if len(names) != 1:
        raise SystemExit(f"kernel substring {kernel!r} matches {names}")

    def main(r):  # the kernel's dispatches; with grid_size, only those of that grid (threads)
        return r["Kernel_Name"] == names[0] and (not grid_size or int(r["Grid_Size"]) == grid_size)
    fetch_k = _counter(fr, "FETCH_SIZE", main)
    write_k = _counter(wr, "WRITE_SIZE", main)
    cf = _counter(fr, "FETCH_SIZE", _copy_rows(fr, "FETCH_SIZE"))
    cw = _counter(wr, "WRITE_SIZE", _copy_rows(wr, "WRITE_SIZE"))
    fetch_factor = COPY_BYTES / (statistics.mean(cf) * 1024)
    write_factor = COPY_BYTES / (statistics.mean(cw) * 1024)
    fetch_b = statistics.mean(fetch_k) * 1024 * fetch_factor
    write_b = statistics.mean(write_k) * 1024 * write_factor
    bench = _last_json(bench_out)
    if entry:  # a secondary workload of the benchmark (full or compact form)
        e = bench["secondary"][entry]
        alg = e["algorithmic_bytes"] if "algorithmic_bytes" in e else e["bytes"]
        workload = f"{entry}: {e['workload']}" if "workload" in e else entry
    else:
        alg = bench["config"]["algorithmic_bytes_per_step"]
        workload = bench["config"]["workload"]
    lines = [
        "# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE and WRITE_SIZE runs),",
        "# each scaled by the same counter's reading for a 1 GiB device copy in the same run.",
        f"# command (FETCH_SIZE; the WRITE_SIZE run differs only in the counter): {command}",
        f"kernel: {names[0]}" + (f" (dispatches with grid size {grid_size} threads)" if grid_size else ""),
        f"workload: {workload}",
        f"library_sha256: {bench['config']['library_sha256']}",
        f"dispatches_fetch: {len(fetch_k)}",
        f"dispatches_write: {len(write_k)}",
        f"fetch_size_kib_per_dispatch: {statistics.mean(fetch_k):.1f}",
        f"write_size_kib_per_dispatch: {statistics.mean(write_k):.1f}",
        f"copy_dispatches: {len(cf)} fetch, {len(cw)} write",
        f"copy_fetch_size_kib_per_GiB: {statistics.mean(cf):.1f}",
        f"copy_write_size_kib_per_GiB: {statistics.mean(cw):.1f}",
        f"fetch_scale: {fetch_factor:.4f}",
        f"write_scale: {write_factor:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / alg:.4f}",
    ]
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--note", action="append", default=[])
    s.add_argument("--trace", default="", help="run_kernel_trace.csv: also split kernels by grid size")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--bench-out", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--entry", default="", help="secondary workload of the benchmark line (default: the main one)")
    t.add_argument("--grid-size", type=int, default=0,
                   help="only the dispatches with this grid size in threads (when workloads share a kernel)")
    a = ap.parse_args(argv)
    text = stats(a.csv, a.command, a.note, a.trace) if a.what == "stats" else traffic(a.fetch, a.write, a.kernel, a.bench_out,
                                                                        a.command, a.entry, a.grid_size)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
