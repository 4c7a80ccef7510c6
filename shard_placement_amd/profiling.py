"""Turn rocprofv3 CSV output into the short text summaries kept under
profiles/ (kernel durations; HBM bytes per launch from FETCH_SIZE and
WRITE_SIZE, scaled by the same counters read on a plain copy of known size).

    python -m shard_placement_amd.profiling stats DIR OUT.txt --command "..."
    python -m shard_placement_amd.profiling pmc FETCH_DIR WRITE_DIR OUT.txt \
        --kernel rs_fixed_kernel --calib-kernel copy --calib-bytes N \
        --algorithmic-bytes B --src-hash H --command "..."
    python -m shard_placement_amd.profiling overlap OUT.txt --dirs D1 D2 \
        --logs L1 L2 --command "..." --title "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
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


def idle_stretches(trace, n: int = 3, names: bool = False):
    """The n longest stretches of a kernel trace with no dispatch running
    (between the end of the last dispatch so far and the start of the
    next), as (length, start, end) in ms from the first dispatch; with
    names=True each also carries the kernel that ended last before the
    stretch and the one that starts it."""
    iv = sorted((int(t["Start_Timestamp"]), int(t["End_Timestamp"]), t.get("Kernel_Name", ""))
                for t in trace)
    if not iv:
        return []
    t0, reach, last, gaps = iv[0][0], iv[0][1], iv[0][2], []
    for a, b, k in iv[1:]:
        if a > reach:
            g = ((a - reach) / 1e6, (reach - t0) / 1e6, (a - t0) / 1e6)
            gaps.append(g + (last, k) if names else g)
        if b >= reach:
            reach, last = b, k
    return sorted(gaps, reverse=True)[:n]


def summarize_stats(d: str, out: str, command: str, top: int = 12, gaps: int = 0) -> None:
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
        if gaps:
            lines.append("")
            lines.append("# the longest stretches with no kernel dispatch running (ms from the first dispatch)")
            for g, a, b, before, after in idle_stretches(tr, gaps, names=True):
                lines.append("no dispatch for %.1f ms: %.3f .. %.3f ms (after %s; before %s)" % (
                    g, a, b, before[:60], after[:60]))
    except FileNotFoundError:
        pass
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _med(xs):
    return statistics.median(xs) if xs else float("nan")


def overlap_of(d: str, gemm_substr: str = "Cijk", rs_substr: str = "rs_fixed_kernel") -> dict:
    """From one process's kernel trace: the GEMMs that overlap at least one
    reduce-scatter launch, their durations, how many launches overlap each
    and how many launch ends fall inside each, the durations of the launches
    that overlap a GEMM and of those that do not (microseconds)."""
    tr = kernel_trace(d)
    span = lambda t: (int(t["Start_Timestamp"]), int(t["End_Timestamp"]))
    gemms = sorted(span(t) for t in tr if gemm_substr in t.get("Kernel_Name", ""))
    rs = sorted(span(t) for t in tr if rs_substr in t.get("Kernel_Name", ""))
    dur, n_ov, n_end, rs_ov = [], [], [], set()
    for a, b in gemms:
        ov = [i for i, (s, e) in enumerate(rs) if s < b and e > a]
        if not ov:
            continue
        dur.append((b - a) / 1e3)
        n_ov.append(len(ov))
        n_end.append(sum(1 for i in ov if a < rs[i][1] < b))
        rs_ov.update(ov)
    rs_ov_d = [(rs[i][1] - rs[i][0]) / 1e3 for i in sorted(rs_ov)]
    rs_free_d = [(e - s) / 1e3 for i, (s, e) in enumerate(rs) if i not in rs_ov]
    return {"gemms": len(dur), "gemm_us": dur, "launches_per_gemm": n_ov,
            "ends_inside": n_end, "rs_overlapping_us": rs_ov_d, "rs_alone_us": rs_free_d}


def summarize_overlap(dirs, logs, out: str, command: str, title: str) -> None:
    """One block per process: the probe's own results (the JSON line that
    bench.py or the standalone probe printed in that process) and the
    overlap figures from its kernel trace."""
    lines = ["# rocprofv3 kernel trace of the default-configuration interference probe, %s" % title,
             "command (one process each): %s" % command,
             "per process: the probe's result line, then over the GEMMs (Cijk_* kernels) that overlap",
             "at least one reduce-scatter launch (rs_fixed_kernel): GEMM duration, launches overlapping",
             "each GEMM, launch ends inside each GEMM, and the duration of the launches that overlap a",
             "GEMM against those that do not"]
    for i, (d, lg) in enumerate(zip(dirs, logs), 1):
        probe = None
        with open(lg) as fh:
            for line in fh:
                if line.startswith("{"):
                    probe = json.loads(line).get("probe")
        o = overlap_of(d)
        lines.append("")
        modes = (probe or {}).get("modes") or []
        for j, m in enumerate(modes):
            lines.append("process %d%s: probe (%s, %s tiles per launch, %s B of LDS per workgroup): RS "
                         "alone %.1f GB/s, beside the GEMM %.1f GB/s; GEMM %.4f -> %s ms (%s%%, %d GEMMs "
                         "inside)" % (
                             i, "" if len(modes) == 1 else " run %d" % (j + 1), m["mode"],
                             m["tiles_per_launch"], m.get("lds_per_workgroup", "?"),
                             m["rs_alone_gbps"],
                             m["rs_concurrent_gbps"], m["t_gemm_alone_ms"],
                             m["t_gemm_concurrent_ms"], m["gemm_slowdown_pct"], m["gemm_inside"]))
        if not o["gemms"]:
            lines.append("  no GEMM overlaps a reduce-scatter launch")
            continue
        lines.append("  GEMMs overlapping the RS: %d; duration median %.0f us (min %.0f, max %.0f)" % (
            o["gemms"], _med(o["gemm_us"]), min(o["gemm_us"]), max(o["gemm_us"])))
        lines.append("  RS launches overlapping each GEMM: median %g (min %d, max %d); launch ends inside "
                     "a GEMM: median %g" % (_med(o["launches_per_gemm"]), min(o["launches_per_gemm"]),
                                            max(o["launches_per_gemm"]), _med(o["ends_inside"])))
        lines.append("  RS launches overlapping a GEMM: %d, duration median %.0f us (max %.0f); the other "
                     "%d: median %.1f us" % (len(o["rs_overlapping_us"]), _med(o["rs_overlapping_us"]),
                                             max(o["rs_overlapping_us"]), len(o["rs_alone_us"]),
                                             _med(o["rs_alone_us"])))
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
    s.add_argument("--gaps", type=int, default=0, help="also list the N longest idle stretches")
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
    o = sub.add_parser("overlap")
    o.add_argument("out")
    o.add_argument("--dirs", nargs="+", required=True, help="kernel-trace folders, one per process")
    o.add_argument("--logs", nargs="+", required=True, help="bench.py output of the same processes")
    o.add_argument("--command", required=True)
    o.add_argument("--title", required=True)
    pp = sub.add_parser("pipeline")
    pp.add_argument("out")
    pp.add_argument("--dirs", nargs="+", required=True, help="kernel-trace folders, one per process")
    pp.add_argument("--logs", nargs="+", required=True, help="output of the same processes")
    pp.add_argument("--command", required=True)
    pp.add_argument("--title", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "pipeline":
        if len(a.dirs) != len(a.logs):
            raise SystemExit("--dirs and --logs must pair up")
        summarize_pipeline(a.dirs, a.logs, a.out, a.command, a.title)
    elif a.cmd == "stats":
        summarize_stats(a.dir, a.out, a.command, gaps=a.gaps)
    elif a.cmd == "overlap":
        if len(a.dirs) != len(a.logs):
            raise SystemExit("--dirs and --logs must pair up")
        summarize_overlap(a.dirs, a.logs, a.out, a.command, a.title)
    else:
        summarize_pmc(a.fetch_dir, a.write_dir, a.out, a.kernel, a.calib_kernel, a.calib_bytes,
                      a.algorithmic_bytes, a.src_hash, a.command_fetch, a.command_write, a.workload)
    return 0



def cu_time(census, stamps, tick_hz: float = 1e8) -> dict:
    """Compute-unit time a reduce-scatter held, from the per-tile trace of
    tide_rs_bf16_to_fp32_trace: census[t] (packed CU id) and stamps[t] =
    (start, end) in real-time counter ticks.  Per CU the union of its tiles'
    intervals is the time it held at least one reduce-scatter workgroup; the
    sum over CUs is the occupancy-weighted CU time (the one-GPU analog of the
    pages' reduce-scatter "SM time").  Also the plain sum of workgroup
    durations and the trace's span.  Inputs are numpy arrays (or anything
    numpy can take)."""
    import numpy as np

    cu = np.asarray(census).astype(np.int64).reshape(-1)
    st = np.asarray(stamps).astype(np.int64).reshape(-1, 2)
    if cu.size == 0:
        return {"cus": 0, "held_cu_ms": 0.0, "workgroup_ms_sum": 0.0, "span_ms": 0.0}
    if np.any(st[:, 1] < st[:, 0]):
        raise ValueError("a tile ends before it starts")
    order = np.lexsort((st[:, 0], cu))
    cu, st = cu[order], st[order]
    held = 0
    bounds = np.flatnonzero(np.diff(cu)) + 1
    for s0, s1 in zip(np.r_[0, bounds], np.r_[bounds, cu.size]):
        a, b = st[s0:s1, 0], st[s0:s1, 1]
        prev_end = np.maximum.accumulate(np.r_[a[0], b[:-1]])
        held += int(np.sum(np.maximum(0, b - np.maximum(a, prev_end))))
    ms = 1e3 / tick_hz
    return {"cus": int(np.unique(cu).size), "held_cu_ms": round(held * ms, 3),
            "workgroup_ms_sum": round(float(np.sum(st[:, 1] - st[:, 0])) * ms, 3),
            "span_ms": round(float(st[:, 1].max() - st[:, 0].min()) * ms, 4),
            "tick_hz": tick_hz}


def workgroup_us_by_xcc(census, stamps, tick_hz: float = 1e8) -> dict:
    """Mean workgroup duration (microseconds) per XCC from the same trace:
    the packed census id carries the XCC in bits [8, 12).  On the MI355X the
    odd-numbered XCCs run the reduce-scatter's workgroups several percent
    longer than the even-numbered ones.  Keys are XCC ids as strings."""
    import numpy as np

    cu = np.asarray(census).astype(np.int64).reshape(-1)
    st = np.asarray(stamps).astype(np.int64).reshape(-1, 2)
    if cu.size == 0:
        return {}
    if np.any(st[:, 1] < st[:, 0]):
        raise ValueError("a tile ends before it starts")
    xcc = (cu >> 8) & 0xF
    dur = (st[:, 1] - st[:, 0]) * (1e6 / tick_hz)
    return {str(int(x)): round(float(dur[xcc == x].mean()), 3) for x in np.unique(xcc)}


def _union(iv):
    """Total length of a union of (start, end) intervals, and the merged list."""
    out, total = [], 0
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    for a, b in out:
        total += b - a
    return total, out


def pipeline_phases(d: str, p1: str = "rs_dense_kernel", p2: str = "rs_drain_kernel") -> dict:
    """From one process's kernel trace of pipelined runs: for the phase-1
    (reduction into staging) and phase-2 (delivery into the arenas)
    dispatches, the hardware queues and streams they ran on, how long each
    phase kept the GPU busy (union of its dispatches), and how long both
    ran at once (microseconds)."""
    tr = kernel_trace(d)
    rows = {1: [], 2: []}
    for t in tr:
        k = t.get("Kernel_Name", "")
        ph = 1 if p1 in k else 2 if p2 in k else 0
        if ph:
            rows[ph].append((int(t["Start_Timestamp"]), int(t["End_Timestamp"]),
                             t.get("Queue_Id"), t.get("Stream_Id")))
    out = {}
    merged = {}
    for ph in (1, 2):
        busy, merged[ph] = _union([(a, b) for a, b, _, _ in rows[ph]])
        out["phase%d" % ph] = {"dispatches": len(rows[ph]),
                               "queues": sorted({q for _, _, q, _ in rows[ph]}),
                               "streams": sorted({s for _, _, _, s in rows[ph]}),
                               "busy_us": round(busy / 1e3, 1)}
    both = 0
    i = j = 0
    m1, m2 = merged[1], merged[2]
    while i < len(m1) and j < len(m2):
        lo, hi = max(m1[i][0], m2[j][0]), min(m1[i][1], m2[j][1])
        if hi > lo:
            both += hi - lo
        if m1[i][1] < m2[j][1]:
            i += 1
        else:
            j += 1
    allr = rows[1] + rows[2]
    span = (max(b for _, b, _, _ in allr) - min(a for a, _, _, _ in allr)) if allr else 0
    out["both_busy_us"] = round(both / 1e3, 1)
    out["span_us"] = round(span / 1e3, 1)
    return out


def summarize_pipeline(dirs, logs, out: str, command: str, title: str) -> None:
    """One block per process: the run's own timing line and the phase
    figures from its kernel trace."""
    lines = ["# rocprofv3 kernel trace of the two-phase pipeline, %s" % title,
             "command (one process each): %s" % command,
             "per process: the pipeline's own timing (events), then from the kernel trace the",
             "hardware queues and streams of phase 1 (rs_dense_kernel) and phase 2",
             "(rs_drain_kernel), each phase's busy time (union of its dispatches), the time both",
             "ran at once, and the span of all of them"]
    for i, (d, lg) in enumerate(zip(dirs, logs), 1):
        res = None
        with open(lg) as fh:
            for line in fh:
                if line.startswith("{"):
                    res = json.loads(line)
        ph = pipeline_phases(d)
        lines.append("")
        lines.append("process %d: %s" % (i, json.dumps(res, sort_keys=True)))
        for k in ("phase1", "phase2"):
            v = ph[k]
            lines.append("  %s: %d dispatches on queues %s, streams %s; busy %.1f us" % (
                k, v["dispatches"], v["queues"], v["streams"], v["busy_us"]))
        lines.append("  both phases at once: %.1f us of a %.1f us span" % (ph["both_busy_us"],
                                                                        ph["span_us"]))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    sys.exit(main())
