"""The rocprofv3 summary writer on synthetic CSVs (CPU): the warm figures
leave out each kernel's first launch, the tail figures keep its last N
launches in launch order, and the traffic figures scale by the copy
kernel's reading."""
import os

from block_sparse_attention_bsattn_amd import rocprof_summary as rs


def _write(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_stats_warm_and_tail(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    # kernel A: launches of 5000, 1000, 2000, 3000, 4000 ns in launch order
    # (written out of order); kernel B: one launch
    durs = [5000, 1000, 2000, 3000, 4000]
    trace = [("A", 100 * i, 100 * i + t) for i, t in enumerate(durs)]
    trace = [trace[i] for i in (3, 0, 4, 1, 2)] + [("B", 50, 1050)]
    _write(d / "x_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    _write(d / "x_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [("A", 5, 15000, 3000, 93.75, 1000, 5000), ("B", 1, 1000, 1000, 6.25, 1000, 1000)])
    text = rs.stats_summary(str(d), "cmd", tail=2)
    line = next(ln for ln in text.splitlines() if ln.rstrip().endswith(" A"))
    cols = line.split()
    # calls, avg, warm avg (1000..4000 -> 2500), warm median (2500), tail avg
    # (last two: 3000, 4000 -> 3500), tail median (3500)
    assert int(cols[0]) == 5
    assert [float(c) for c in cols[1:6]] == [3.0, 2.5, 2.5, 3.5, 3.5]
    line_b = next(ln for ln in text.splitlines() if ln.rstrip().endswith(" B"))
    assert "n/a" in line_b.split()[2]  # no launch after B's first


def test_traffic_scales_by_the_copy(tmp_path):
    fd, wd = tmp_path / "f", tmp_path / "w"
    fd.mkdir()
    wd.mkdir()
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # the copy of 1 MiB reads as 512 KiB of FETCH_SIZE and 1024 KiB of
    # WRITE_SIZE; the kernel reads 300 and 200 KiB in two launches
    _write(fd / "f_counter_collection.csv", hdr,
           [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0),
            (2, "kern<x>", "FETCH_SIZE", 300.0), (3, "kern<x>", "FETCH_SIZE", 200.0)])
    _write(wd / "w_counter_collection.csv", hdr,
           [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0),
            (2, "kern<x>", "WRITE_SIZE", 64.0), (3, "kern<x>", "WRITE_SIZE", 64.0)])
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    text = rs.traffic_summary(str(fd), str(wd), "kern", 1.0, str(src), "cf", "cw")
    vals = dict(ln.split(": ", 1) for ln in text.splitlines() if ": " in ln)
    assert float(vals["fetch_scale"]) == 2.0 and float(vals["write_scale"]) == 1.0
    # (300 + 200) / 2 KiB x 2 = 500 KiB; writes 64 KiB
    assert int(vals["fetch_bytes_per_launch"]) == 500 * 1024
    assert int(vals["write_bytes_per_launch"]) == 64 * 1024
    assert rs.read_traffic(str(tmp_path / "none.txt"), str(src)) is None
    out = tmp_path / "t.txt"
    out.write_text(text)
    assert rs.read_traffic(str(out), str(src)) is not None
    src.write_text("// changed\n")
    assert rs.read_traffic(str(out), str(src)) is None


def test_l2_hit_rate(tmp_path):
    d = tmp_path / "l2"
    d.mkdir()
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # two launches: 75 % and 50 % hits; another kernel is ignored
    _write(d / "l2_counter_collection.csv", hdr,
           [(1, "kern<x>", "TCC_HIT_sum", 300.0), (1, "kern<x>", "TCC_MISS_sum", 100.0),
            (2, "kern<x>", "TCC_HIT_sum", 50.0), (2, "kern<x>", "TCC_MISS_sum", 50.0),
            (3, "other", "TCC_HIT_sum", 0.0), (3, "other", "TCC_MISS_sum", 10.0)])
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    text = rs.l2_summary(str(d), "kern", str(src), "cmd")
    kv = dict(ln.split(": ", 1) for ln in text.splitlines() if ": " in ln)
    assert kv["launches"] == "2"
    assert float(kv["l2_hit_rate_mean"]) == 0.625
    assert float(kv["l2_hit_rate_min"]) == 0.5 and float(kv["l2_hit_rate_max"]) == 0.75
    assert float(kv["l2_requests_per_launch"]) == 250.0


def test_stats_reports_the_same_runs_bench_line(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    _write(d / "x_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [("A", 0, 1000), ("A", 2000, 3000)])
    _write(d / "x_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [("A", 2, 2000, 1000, 100.0, 1000, 1000)])
    log = tmp_path / "bench.log"
    log.write_text("profiler noise\n{not json}\n"
                   '{"value": 5.0, "unit": "TFLOP/s", "ms_per_step": 1.1, '
                   '"roofline": {"kernel": "A", "fwd_ms_mean": 1.0, "frac": 0.5}}\n')
    text = rs.stats_summary(str(d), "cmd", bench_log=str(log))
    assert "fwd_ms_mean: 1.0" in text and "roofline_frac: 0.5" in text
    assert "ms_per_step: 1.1" in text
