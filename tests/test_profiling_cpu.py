"""The rocprofv3 summary helpers on hand-made traces (CPU)."""
import csv
import json

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
