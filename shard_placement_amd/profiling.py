"""Turn rocprofv3 CSV output into the short text summaries kept under
profiles/ (kernel durations; HBM bytes per launch from FETCH_SIZE and
WRITE_SIZE, scaled by the same counters read on a plain copy of known size).

    python -m shard_placement_amd.profiling stats DIR OUT.txt --command "..."
    python -m shard_placement_amd.profiling pmc FETCH_DIR WRITE_DIR OUT.txt \
        --kernel rs_fixed_kernel --calib-kernel copy --calib-bytes N \
        --algorithmic-bytes B --src-hash H --command "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[-1]


def kernel_stats(d: str):
    rows = []
    with open(_find(d, "kernel_stats.csv")) as fh:
        for row in csv.DictReader(fh):
            rows.append(row)
    return rows


def kernel_trace(d: str):
    with open(_find(d, "kernel_trace.csv")) as fh:
        return list(csv.DictReader(fh))


def summarize_stats(d: str, out: str, command: str, top: int = 12) -> None:
    rows = kernel_stats(d)
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    lines = ["# rocprofv3 kernel statistics", "command: %s" % command,
             "%-70s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    for r in rows[:top]:
        name = r["Name"][:70]
        lines.append("%-70s %6s %12.2f %12.2f %12.2f" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    try:
        tr = kernel_trace(d)
        seen = {}
        for t in tr:
            k = t.get("Kernel_Name", "")
            if k not in seen:
                seen[k] = t
        lines.append("")
        lines.append("# launch shapes (first dispatch of each kernel)")
        for k, t in list(seen.items())[:top]:
            lines.append("%-70s grid=%s wg=%s vgpr=%s sgpr=%s lds=%s scratch=%s" % (
                k[:70], t.get("Grid_Size", t.get("Grid_Size_X", "?")),
                t.get("Workgroup_Size", t.get("Workgroup_Size_X", "?")),
                t.get("VGPR_Count", t.get("Arch_VGPR_Count", "?")), t.get("SGPR_Count", "?"),
                t.get("LDS_Block_Size", t.get("Lds_Size", "?")),
                t.get("Scratch_Size", "?")))
    except FileNotFoundError:
        pass
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counter_per_dispatch(d: str, counter: str, kernel_substr: str):
    vals = []
    with open(_find(d, "counter_collection.csv")) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            if kernel_substr not in row.get("Kernel_Name", ""):
                continue
            vals.append(float(row["Counter_Value"]))
    return vals


def summarize_pmc(fetch_dir, write_dir, out, kernel, calib_kernel, calib_bytes,
                  algorithmic_bytes, src_hash, command_fetch, command_write, workload):
    f = counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    w = counter_per_dispatch(write_dir, "WRITE_SIZE", kernel)
    cf = counter_per_dispatch(fetch_dir, "FETCH_SIZE", calib_kernel)
    cw = counter_per_dispatch(write_dir, "WRITE_SIZE", calib_kernel)
    if not (f and w and cf and cw):
        raise SystemExit("missing dispatches: %d %d %d %d" % (len(f), len(w), len(cf), len(cw)))
    kib = 1024.0
    fetch = statistics.median(f) * kib
    write = statistics.median(w) * kib
    kf = calib_bytes / (statistics.median(cf) * kib)
    kw = calib_bytes / (statistics.median(cw) * kib)
    hbm = fetch * kf + write * kw
    lines = [
        "# rocprofv3 counters (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) for %s on %s" % (kernel, workload),
        "command_fetch: %s" % command_fetch,
        "command_write: %s" % command_write,
        "kernel: %s" % kernel,
        "workload: %s" % workload,
        "kernel_code_sha256_16 (comments stripped): %s" % src_hash,
        "dispatches_fetch: %d" % len(f),
        "dispatches_write: %d" % len(w),
        "fetch_kib_median: %.1f" % (fetch / kib),
        "write_kib_median: %.1f" % (write / kib),
        "calib_kernel: %s (plain device copy of %d bytes)" % (calib_kernel, calib_bytes),
        "calib_fetch_kib: %.1f" % statistics.median(cf),
        "calib_write_kib: %.1f" % statistics.median(cw),
        "calib_factor_fetch: %.4f" % kf,
        "calib_factor_write: %.4f" % kw,
        "hbm_read_bytes_per_launch: %.0f" % (fetch * kf),
        "hbm_write_bytes_per_launch: %.0f" % (write * kw),
        "hbm_bytes_per_launch: %.0f" % hbm,
        "algorithmic_bytes_per_launch: %d" % algorithmic_bytes,
        "traffic_over_algorithmic: %.4f" % (hbm / algorithmic_bytes),
    ]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("out")
    p.add_argument("--kernel", required=True)
    p.add_argument("--calib-kernel", required=True)
    p.add_argument("--calib-bytes", type=int, required=True)
    p.add_argument("--algorithmic-bytes", type=int, required=True)
    p.add_argument("--src-hash", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--command-fetch", required=True)
    p.add_argument("--command-write", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        summarize_stats(a.dir, a.out, a.command)
    else:
        summarize_pmc(a.fetch_dir, a.write_dir, a.out, a.kernel, a.calib_kernel, a.calib_bytes,
                      a.algorithmic_bytes, a.src_hash, a.command_fetch, a.command_write, a.workload)
    return 0


if __name__ == "__main__":
    sys.exit(main())
