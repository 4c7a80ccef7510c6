"""The rocprofv3 summary helpers on hand-made traces (CPU)."""
import csv
import json

import pytest

from shard_placement_amd import profiling


def _trace(tmp_path, rows):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, s, e in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": s, "End_Timestamp": e})
    return str(d)


def test_overlap_counts(tmp_path):
    rs = "void rs_fixed_kernel<8, true, 1, true, true>(...)"
    gemm = "Cijk_Ailk_Bljk_BBS_MT256x256x64"
    rows = [(rs, 0, 45_000), (rs, 46_000, 91_000),        # alone
            (gemm, 100_000, 300_000),                       # overlaps launches 3 and 4
            (rs, 92_000, 310_000), (rs, 311_000, 356_000),
            (gemm, 301_000, 330_000),                        # overlaps launches 3 and 4
            (gemm, 400_000, 500_000)]                        # overlaps nothing
    o = profiling.overlap_of(_trace(tmp_path, rows))
    assert o["gemms"] == 2
    assert o["gemm_us"] == [200.0, 29.0]
    assert o["launches_per_gemm"] == [1, 2]
    assert o["ends_inside"] == [0, 1]
    assert sorted(o["rs_overlapping_us"]) == [45.0, 218.0]
    assert sorted(o["rs_alone_us"]) == [45.0, 45.0]


def test_overlap_summary_reads_the_probe_line(tmp_path):
    rs, gemm = "rs_fixed_kernel<8>", "Cijk_x"
    d = _trace(tmp_path, [(rs, 0, 50_000), (gemm, 10_000, 230_000), (rs, 51_000, 240_000)])
    log = tmp_path / "bench.log"
    mode = {"mode": "default", "tiles_per_launch": 512, "rs_alone_gbps": 6000.0,
            "rs_concurrent_gbps": 5000.0, "t_gemm_alone_ms": 0.205, "t_gemm_concurrent_ms": 0.22,
            "gemm_slowdown_pct": 7.3, "gemm_inside": 40}
    log.write_text("[bench] x\n" + json.dumps({"probe": {"modes": [mode]}}) + "\n")
    out = tmp_path / "s.txt"
    profiling.summarize_overlap([d], [str(log)], str(out), "cmd", "a layer")
    text = out.read_text()
    assert "512 tiles per launch, ? B of LDS per workgroup" in text and "(7.3%, 40 GEMMs inside)" in text
    assert "GEMMs overlapping the RS: 1; duration median 220 us" in text
    assert "launch ends inside a GEMM: median 1" in text


def test_cu_time_union_per_cu():
    from shard_placement_amd.profiling import cu_time

    # CU 1: [0,10) and [5,20) overlap -> 20 ticks held; [30,35) -> 5 more
    # CU 2: [0,4), [4,8) touch -> 8; nested [1,3) adds nothing
    census = [1, 2, 1, 2, 1, 2]
    stamps = [[0, 10], [0, 4], [5, 20], [4, 8], [30, 35], [1, 3]]
    r = cu_time(census, stamps, tick_hz=1e3)  # 1 tick = 1 ms
    assert r["cus"] == 2
    assert r["held_cu_ms"] == 33.0
    assert r["workgroup_ms_sum"] == 10 + 4 + 15 + 4 + 5 + 2
    assert r["span_ms"] == 35.0


def test_cu_time_rejects_reversed_intervals():
    import pytest

    from shard_placement_amd.profiling import cu_time

    with pytest.raises(ValueError):
        cu_time([0], [[5, 4]])


def test_workgroup_us_by_xcc():
    from shard_placement_amd.profiling import workgroup_us_by_xcc

    # tiles on XCC 0 (ids 0x005, 0x00a) last 10 and 20 ticks, on XCC 3
    # (id 0x301) 40 ticks; 1 tick = 1 us
    census = [0x005, 0x301, 0x00A]
    stamps = [[0, 10], [5, 45], [100, 120]]
    assert workgroup_us_by_xcc(census, stamps, tick_hz=1e6) == {"0": 15.0, "3": 40.0}
    assert workgroup_us_by_xcc([], []) == {}
    with pytest.raises(ValueError):
        workgroup_us_by_xcc([0], [[5, 4]])


def test_pipeline_phases_from_a_trace(tmp_path):
    """Queues, busy time and time-both-busy from a made-up kernel trace."""
    from shard_placement_amd.profiling import pipeline_phases

    d = tmp_path / "run"
    d.mkdir()
    rows = [("rs_dense_kernel<8>", 3, 11, 0, 100), ("rs_drain_kernel<true>", 4, 12, 90, 150),
            ("rs_dense_kernel<8>", 3, 11, 100, 200), ("rs_drain_kernel<true>", 4, 12, 200, 260),
            ("Cijk_gemm", 1, 0, 0, 500)]
    with open(d / "run_kernel_trace.csv", "w") as fh:
        fh.write('"Kind","Queue_Id","Stream_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for k, q, s, a, b in rows:
            fh.write('"KERNEL_DISPATCH",%d,%d,"%s",%d,%d\n' % (q, s, k, a * 1000, b * 1000))
    r = pipeline_phases(str(d))
    assert r["phase1"] == {"dispatches": 2, "queues": ["3"], "streams": ["11"], "busy_us": 200.0}
    assert r["phase2"] == {"dispatches": 2, "queues": ["4"], "streams": ["12"], "busy_us": 120.0}
    assert r["both_busy_us"] == 60.0 and r["span_us"] == 260.0


def test_idle_stretches():
    from shard_placement_amd.profiling import idle_stretches

    ms = 1_000_000
    tr = [{"Start_Timestamp": a * ms, "End_Timestamp": b * ms}
          for a, b in [(0, 10), (5, 12), (40, 50), (50, 51), (200, 210), (60, 70)]]
    assert idle_stretches(tr, 2) == [(130.0, 70.0, 200.0), (28.0, 12.0, 40.0)]
    assert idle_stretches([], 3) == []
    for i, t in enumerate(tr):
        t["Kernel_Name"] = "k%d" % i
    # the stretch 70..200 follows k5 (ends at 70) and precedes k4; 12..40
    # follows k1 (the later end of the overlapping pair) and precedes k2
    assert idle_stretches(tr, 2, names=True) == [(130.0, 70.0, 200.0, "k5", "k4"),
                                                 (28.0, 12.0, 40.0, "k1", "k2")]
