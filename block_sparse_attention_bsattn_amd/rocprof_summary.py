"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

Three summaries:

  stats    per-kernel call count and durations from a ``--kernel-trace
           --stats`` run (the ``*_kernel_stats.csv`` file), with the mean and
           median over every launch after a kernel's first from the
           per-dispatch trace (``*_kernel_trace.csv``), and with ``--tail N``
           over each kernel's last N launches;
  mfma     the matrix-core busy fraction and executed bf16 MFMA work of one
           kernel from one ``--pmc`` run (SQ_VALU_MFMA_BUSY_CYCLES,
           GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_BF16);
  traffic  HBM bytes per launch of one kernel from two ``--pmc`` runs, one
           with FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch).  Both
           counters are scaled by what they read for a plain device copy of
           known size in the same run (the largest ``__amd_rocclr_copyBuffer``
           dispatch: it reads and writes ``copy_mib`` MiB).

The traffic summary records the SHA-256 of the kernel's source file; a reader
(bench.py) uses the figures only while the source still hashes the same.

Usage:
  python -m block_sparse_attention_bsattn_amd.rocprof_summary stats \\
      --csv-dir DIR --command "..." --out profiles/NAME.txt
  python -m block_sparse_attention_bsattn_amd.rocprof_summary traffic \\
      --fetch-dir DIR --write-dir DIR --kernel SUBSTR --copy-mib 256 \\
      --source FILE --command-fetch "..." --command-write "..." --out FILE
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(f"no file matches {pattern}")
    return hits[-1]


def source_sha256(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _dispatch_durations(csv_dir: str):
    """{kernel name: [duration ns of each dispatch, in launch order]} from the
    per-dispatch kernel trace, or {} when the trace is missing."""
    try:
        path = _one(os.path.join(csv_dir, "**", "*kernel_trace.csv"))
    except FileNotFoundError:
        return {}
    per: dict = {}
    for r in csv.DictReader(open(path)):
        if not {"Kernel_Name", "Start_Timestamp", "End_Timestamp"} <= r.keys():
            return {}
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, lst in per.items():
        lst.sort()
        out[name] = [d for _, d in lst]
    return out


def _bench_line(path: str):
    """The last JSON line a benchmark run printed (None if there is none)."""
    import json
    last = None
    for line in open(path, errors="replace"):
        line = line.strip()
        if line.startswith("{") and line.endswith("}"):
            try:
                last = json.loads(line)
            except ValueError:
                pass
    return last


def stats_summary(csv_dir: str, command: str, top: int = 12, tail: int = 0,
                  bench_log: str = "") -> str:
    """The kernel statistics, with the mean and median over every launch
    after a kernel's first (the first pays one-time costs: code object load,
    cold caches) and, with tail > 0, over each kernel's last `tail` launches
    (a benchmark's timed steps, when its warm-up steps come first).  With
    bench_log, the forward time the same run's benchmark line reports from
    its own events, to compare with the traced durations."""
    path = _one(os.path.join(csv_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    disp = _dispatch_durations(csv_dir)
    lines = ["# rocprofv3 kernel-trace statistics", "",
             f"command: {command}", "",
             "warm_avg_us / warm_med_us: every launch after a kernel's first "
             "(from the per-dispatch trace)"]
    if tail > 0:
        lines.append(f"tail_avg_us / tail_med_us: each kernel's last {tail} launches "
                     "(the timed steps)")
    lines += ["", f"{'calls':>6} {'avg_us':>10} {'warm_avg_us':>12} {'warm_med_us':>12} "
              + (f"{'tail_avg_us':>12} {'tail_med_us':>12} " if tail > 0 else "")
              + f"{'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}  kernel"]
    fmt = lambda f, xs: f"{f(xs) / 1e3:12.2f}" if xs else f"{'n/a':>12}"
    for r in rows[:top]:
        name = r["Name"]
        d = disp.get(name, [])
        wd, td = d[1:], d[-tail:] if tail > 0 else []
        extra = (fmt(statistics.mean, td) + " " + fmt(statistics.median, td) + " "
                 if tail > 0 else "")
        wa, wm = fmt(statistics.mean, wd), fmt(statistics.median, wd)
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {wa} {wm} {extra}"
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f} "
                     f"{float(r['Percentage']):6.2f}  {name}")
    if bench_log:
        b = _bench_line(bench_log)
        if b is not None and b.get("roofline"):
            rf = b["roofline"]
            lines += ["", "same run, benchmark line (HIP events on the launch stream):",
                      f"  kernel: {rf.get('kernel')}",
                      f"  fwd_ms_mean: {rf.get('fwd_ms_mean')}",
                      f"  roofline_frac: {rf.get('frac')}",
                      f"  ms_per_step: {b.get('ms_per_step')}",
                      f"  value: {b.get('value')} {b.get('unit')}"]
    return "\n".join(lines) + "\n"


def _counter_by_dispatch(csv_dir: str, counter: str):
    """{kernel name: [(dispatch id, value), ...]} for one counter."""
    path = _one(os.path.join(csv_dir, "**", "*counter_collection.csv"))
    out: dict = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return out


def _kernel_values(per: dict, substr: str):
    vals = [v for name, dv in per.items() if substr in name for _, v in dv]
    if not vals:
        raise KeyError(f"no dispatch of a kernel matching {substr!r}")
    return vals


def traffic_summary(fetch_dir, write_dir, kernel, copy_mib, source,
                    command_fetch, command_write):
    fetch = _counter_by_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_by_dispatch(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_copy = max(_kernel_values(fetch, COPY_KERNEL))
    w_copy = max(_kernel_values(write, COPY_KERNEL))
    f_scale = copy_kib / f_copy
    w_scale = copy_kib / w_copy
    kf = _kernel_values(fetch, kernel)
    kw = _kernel_values(write, kernel)
    f_bytes = statistics.mean(kf) * f_scale * 1024.0
    w_bytes = statistics.mean(kw) * w_scale * 1024.0
    lines = [
        "# HBM traffic per launch from rocprofv3 PMC counters", "",
        f"kernel: {kernel}",
        f"source: {os.path.relpath(source)}",
        f"source_sha256: {source_sha256(source)}",
        f"command_fetch: {command_fetch}",
        f"command_write: {command_write}",
        f"copy_calibration_mib: {copy_mib}",
        f"copy_fetch_kib_measured: {f_copy:.1f}",
        f"copy_write_kib_measured: {w_copy:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"launches_fetch: {len(kf)}",
        f"launches_write: {len(kw)}",
        f"fetch_kib_raw_mean: {statistics.mean(kf):.1f}",
        f"write_kib_raw_mean: {statistics.mean(kw):.1f}",
        f"fetch_bytes_per_launch: {f_bytes:.0f}",
        f"write_bytes_per_launch: {w_bytes:.0f}",
        f"traffic_bytes_per_launch: {f_bytes + w_bytes:.0f}",
    ]
    return "\n".join(lines) + "\n"


def read_traffic(path: str, source: str):
    """The traffic summary as a dict, or None when it is missing or was taken
    on a different version of the kernel source."""
    if not os.path.exists(path) or not os.path.exists(source):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha256(source):
        return None
    return {"fetch": float(kv["fetch_bytes_per_launch"]),
            "write": float(kv["write_bytes_per_launch"]),
            "total": float(kv["traffic_bytes_per_launch"])}


def mfma_summary(pmc_dir, kernel, simds, xcds, source, command):
    """Matrix-core busy fraction per launch of one kernel: the summed
    SQ_VALU_MFMA_BUSY_CYCLES of all SIMDs over (kernel cycles x SIMDs), the
    MfmaUtil expression rocprofv3 lists.  The CSV's GRBM_GUI_ACTIVE is the
    sum over the XCDs' instances (about 8 x the kernel's cycles), so the
    kernel's cycles are that sum / xcds.  Also the bf16 MFMA work executed
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOPs)."""
    busy = dict(_counter_by_dispatch(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES"))
    gui = dict(_counter_by_dispatch(pmc_dir, "GRBM_GUI_ACTIVE"))
    mops = dict(_counter_by_dispatch(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
    utils, flops = [], []
    for name, dv in busy.items():
        if kernel not in name:
            continue
        g = {d: v for d, v in gui.get(name, [])}
        m = {d: v for d, v in mops.get(name, [])}
        for d, b in dv:
            if g.get(d):
                utils.append(b / (g[d] / xcds * simds))
            if d in m:
                flops.append(m[d] * 512.0)
    if not utils:
        raise KeyError(f"no dispatch of a kernel matching {kernel!r}")
    lines = [
        "# Matrix-core busy fraction from rocprofv3 PMC counters", "",
        f"kernel: {kernel}",
        f"source: {os.path.relpath(source)}",
        f"source_sha256: {source_sha256(source)}",
        f"command: {command}",
        "counters: SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs), GRBM_GUI_ACTIVE, "
        "SQ_INSTS_VALU_MFMA_MOPS_BF16",
        f"simds: {simds}",
        f"xcds (GRBM_GUI_ACTIVE instances summed in the CSV): {xcds}",
        f"launches: {len(utils)}",
        f"mfma_busy_fraction_mean: {statistics.mean(utils):.4f}",
        f"mfma_busy_fraction_min: {min(utils):.4f}",
        f"mfma_busy_fraction_max: {max(utils):.4f}",
        f"bf16_mfma_flops_per_launch: {statistics.mean(flops):.4e}" if flops else
        "bf16_mfma_flops_per_launch: n/a",
    ]
    return "\n".join(lines) + "\n"


def l2_summary(pmc_dir, kernel, source, command):
    """L2 hit rate per launch of one kernel: TCC_HIT_sum / (TCC_HIT_sum +
    TCC_MISS_sum), both summed over the L2 channels of every XCD."""
    hit = dict(_counter_by_dispatch(pmc_dir, "TCC_HIT_sum"))
    miss = dict(_counter_by_dispatch(pmc_dir, "TCC_MISS_sum"))
    rates, reqs = [], []
    for name, dv in hit.items():
        if kernel not in name:
            continue
        m = {d: v for d, v in miss.get(name, [])}
        for d, h in dv:
            if d in m and h + m[d] > 0:
                rates.append(h / (h + m[d]))
                reqs.append(h + m[d])
    if not rates:
        raise KeyError(f"no dispatch of a kernel matching {kernel!r}")
    lines = [
        "# L2 hit rate from rocprofv3 PMC counters", "",
        f"kernel: {kernel}",
        f"source: {os.path.relpath(source)}",
        f"source_sha256: {source_sha256(source)}",
        f"command: {command}",
        "counters: TCC_HIT_sum, TCC_MISS_sum (all L2 channels of all XCDs)",
        f"launches: {len(rates)}",
        f"l2_hit_rate_mean: {statistics.mean(rates):.4f}",
        f"l2_hit_rate_min: {min(rates):.4f}",
        f"l2_hit_rate_max: {max(rates):.4f}",
        f"l2_requests_per_launch: {statistics.mean(reqs):.4e}",
    ]
    return "\n".join(lines) + "\n"


def read_mfma(path: str, source: str):
    """The MFMA summary as a dict, or None when missing or taken on another
    version of the kernel source."""
    if not os.path.exists(path) or not os.path.exists(source):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha256(source):
        return None
    out = {"busy": float(kv["mfma_busy_fraction_mean"])}
    f = kv.get("bf16_mfma_flops_per_launch", "n/a")
    out["flops"] = None if f == "n/a" else float(f)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv-dir", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--tail", type=int, default=0)
    s.add_argument("--bench-log", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-dir", required=True)
    t.add_argument("--write-dir", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--pmc-dir", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--source", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--out", required=True)
    c = sub.add_parser("l2")
    c.add_argument("--pmc-dir", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--source", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        text = stats_summary(a.csv_dir, a.command, tail=a.tail, bench_log=a.bench_log)
    elif a.cmd == "l2":
        text = l2_summary(a.pmc_dir, a.kernel, a.source, a.command)
    elif a.cmd == "mfma":
        text = mfma_summary(a.pmc_dir, a.kernel, a.simds, a.xcds, a.source, a.command)
    else:
        text = traffic_summary(a.fetch_dir, a.write_dir, a.kernel, a.copy_mib,
                               a.source, a.command_fetch, a.command_write)
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
