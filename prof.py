"""Summaries of rocprofv3 runs of bench.py: per-kernel durations and HBM traffic,
and issue counters.

Usage (paths are the rocprofv3 output directories of one command each):
  python prof.py --trace DIR --fetch DIR --write DIR \\
      --workload NAME --path one --command "..." --out profiles/NAME.md
  python prof.py counters DIR [DIR ...] --title "..." --command "..." [--command ...] \\
      --build B --out profiles/NAME.md

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
counters read for a kernel of known traffic (bench.py --calibrate-copy: four
dispatches of the probe kernel, each reading 256 MiB and writing 256 MiB), so
that the reported traffic is in bytes of HBM reads and writes.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

COPY_BYTES = 256 << 20


def write_atomic(path, text):
    """Write text to path through a temporary file and a rename, so that a
    reader never sees a half-written file."""
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        f.write(text)
    os.replace(tmp, path)


def _csv(d, suffix):
    f = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not f:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(f[0])))


def kernel_stats(trace_dir):
    """Average/min/max/count of each kernel's duration (ns) from the kernel trace."""
    rows = _csv(trace_dir, "kernel_trace.csv")
    by = {}
    for r in rows:
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by.setdefault(r["Kernel_Name"], []).append(d)
    return {k: {"count": len(v), "avg_ns": statistics.mean(v), "median_ns": statistics.median(v),
                "min_ns": min(v), "max_ns": max(v)} for k, v in by.items()}


def last_dispatches(trace_dir, n):
    """Durations of the last n dispatches of the library's kernels, their mean
    start-to-start spacing and the idle time between one kernel's end and the
    next one's start, as markdown lines."""
    rows = [r for r in _csv(trace_dir, "kernel_trace.csv") if "arrms::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rows = rows[-n:]
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    st = [int(r["Start_Timestamp"]) for r in rows]
    en = [int(r["End_Timestamp"]) for r in rows]
    gaps = [(st[i + 1] - en[i]) / 1e3 for i in range(len(rows) - 1)]
    out = [f"- `{k[:90]}`: {len(v)} dispatches, mean {statistics.mean(v):.3f} us, median {statistics.median(v):.3f} us"
           for k, v in by.items()]
    out.append(f"- start-to-start spacing: mean {(st[-1] - st[0]) / 1e3 / (len(rows) - 1):.3f} us")
    out.append(f"- idle between one kernel's end and the next one's start: median {statistics.median(gaps):.3f} us, "
               f"mean {statistics.mean(gaps):.3f} us")
    return out


def counter(dir_, name):
    rows = _csv(dir_, "counter_collection.csv")
    by = {}
    for r in rows:
        if r["Counter_Name"] == name:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return by


def calibration_kernel(names):
    """The calibration kernel (bench.py --calibrate-copy: the probe kernel, each
    dispatch reading and writing COPY_BYTES), or None."""
    for n in names:
        if "probe_kernel" in n:
            return n
    return None


def counter_medians(dirs):
    """{kernel: {counter: median over its dispatches}} over rocprofv3 --pmc output
    directories (one counter set each), for the library's kernels."""
    out = {}
    for d in dirs:
        by = {}
        for r in _csv(d, "counter_collection.csv"):
            if "arrms::" not in r["Kernel_Name"]:
                continue
            by.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        for (k, c), v in by.items():
            out.setdefault(k, {})[c] = statistics.median(v)
    return out


def derived(cs):
    """Per-wave and per-cycle figures from the issue counters (whichever are there)."""
    d = {}
    w = cs.get("SQ_WAVES")
    if w:
        for c, name in (("SQ_INSTS_VALU", "VALU instructions per wave"), ("SQ_INSTS_SALU", "SALU instructions per wave"),
                        ("SQ_INSTS_VMEM_RD", "vector memory reads per wave"),
                        ("SQ_INSTS_VMEM_WR", "vector memory writes per wave"),
                        ("SQ_WAVE_CYCLES", "wave lifetime, cycles")):
            if c in cs:
                d[name] = cs[c] / w
    wc = cs.get("SQ_WAVE_CYCLES")
    if wc:
        for c, name in (("SQ_WAIT_INST_ANY", "share of wave cycles waiting for an issue slot"),
                        ("SQ_WAIT_ANY", "share of wave cycles waiting on memory or a dependency")):
            if c in cs:
                d[name] = cs[c] / wc
    return d


def counters_main(argv):
    ap = argparse.ArgumentParser(prog="prof.py counters",
                                 description="Median issue counters of the library's kernels, one pass per directory")
    ap.add_argument("dirs", nargs="+", help="rocprofv3 --pmc output directories")
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", action="append", required=True,
                    help="the profiled command of each pass, in the order of dirs")
    ap.add_argument("--build", required=True, help="first 16 hex digits of the SHA-256 of libarrms.so")
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    med = counter_medians(a.dirs)
    kernels = sorted(med)
    names = sorted({c for k in kernels for c in med[k]})
    lines = [f"# rocprofv3 counters: {a.title}", "", "One counter pass per run (run from the repository root):", "",
             "```"] + a.command + ["```", "", f"Library build (SHA-256 of libarrms.so, first 16 hex digits): `{a.build}`. "
             "Values: median over the "
             "dispatches of each kernel of the counter summed over the device's instances. Under counter collection "
             "kernels run slower than in bench.py, so cycle counts are compared per wave and as ratios, not as times.",
             "", "| counter | " + " | ".join(f"`{k[:60]}`" for k in kernels) + " |",
             "|---|" + "---|" * len(kernels)]
    for c in names:
        lines.append(f"| {c} | " + " | ".join(f"{med[k].get(c, float('nan')):.0f}" for k in kernels) + " |")
    lines += ["", "Derived:", ""]
    for k in kernels:
        dv = derived(med[k])
        lines.append(f"- `{k[:60]}`: " + "; ".join(f"{n} {v:.3f}" if n.startswith("share") else f"{n} {v:.1f}"
                                                  for n, v in dv.items()))
    write_atomic(a.out, "\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        counters_main(sys.argv[2:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output (omit for a trace-only summary)")
    ap.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output")
    ap.add_argument("--last", type=int, default=0,
                    help="also summarise the last N dispatches of the library's kernels (the end of the timed "
                         "part of the run): durations, start-to-start spacing, idle gap between kernels")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--path", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--build", required=True, help="the library build profiled: first 16 hex digits of the "
                    "SHA-256 of libarrms.so (bench.library_build())")
    ap.add_argument("--algo-bytes", type=int, required=True)
    ap.add_argument("--bench-us", type=float, required=True, help="bench.py us/call of the same command")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json")
    a = ap.parse_args()

    ks = kernel_stats(a.trace)
    fetch = counter(a.fetch, "FETCH_SIZE") if a.fetch else {}
    write = counter(a.write, "WRITE_SIZE") if a.write else {}
    ck = calibration_kernel(fetch)
    # each calibration dispatch reads and writes COPY_BYTES
    f_copy = statistics.mean(fetch[ck]) if ck else None
    w_copy = statistics.mean(write[ck]) if ck and write.get(ck) else None
    f_scale = COPY_BYTES / (f_copy * 1024.0) if f_copy else None
    w_scale = COPY_BYTES / (w_copy * 1024.0) if w_copy else None
    ours = [k for k in ks if "arrms::" in k]
    lines = [f"# rocprofv3 summary: {a.workload}, path {a.path}", "",
             "Command (run from the repository root, one run per block below):", "",
             "```", f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- {a.command}"] + \
            ([f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- {a.command}",
              f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- {a.command}"] if a.fetch else []) + \
            ["```", "",
             f"Library build (SHA-256 of libarrms.so, first 16 hex digits): `{a.build}`. bench.py us/call of the "
             f"same command, under the profiler "
             f"(which adds its own cost to every launch): {a.bench_us:.3f}.",
             "", "| kernel | dispatches | avg us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for k in sorted(ks, key=lambda k: -ks[k]["avg_ns"] * ks[k]["count"]):
        v = ks[k]
        lines.append(f"| `{k[:90]}` | {v['count']} | {v['avg_ns']/1e3:.3f} | {v['median_ns']/1e3:.3f} | "
                     f"{v['min_ns']/1e3:.3f} | {v['max_ns']/1e3:.3f} |")
    if a.last:
        lines += ["", f"The last {a.last} dispatches of the library's kernels (the end of the timed part of the "
                  "run):", ""] + last_dispatches(a.trace, a.last)
    if not a.fetch:
        write_atomic(a.out, "\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    lines += ["", "HBM traffic per dispatch (counter KiB scaled by the calibration kernel's reading):", ""]
    if ck:
        lines.append(f"- calibration kernel `{ck[:60]}` ({len(fetch[ck])} dispatches, each reading and writing "
                     f"256 MiB): FETCH_SIZE {f_copy:.0f} KiB, WRITE_SIZE {w_copy:.0f} KiB per dispatch -> scale "
                     f"factors {f_scale:.4f} (reads), {w_scale:.4f} (writes)")
    traffic = {}
    for k in ours:
        if k not in fetch:
            continue
        fr = statistics.mean(fetch[k]) * 1024.0 * (f_scale or 1.0)
        wr = statistics.mean(write.get(k, [0.0])) * 1024.0 * (w_scale or 1.0)
        lines.append(f"- `{k[:90]}`: reads {fr/1e6:.2f} MB, writes {wr/1e6:.2f} MB, total {(fr+wr)/1e6:.2f} MB "
                     f"(algorithmic {a.algo_bytes/1e6:.2f} MB per call)")
        traffic[k] = fr + wr
    write_atomic(a.out, "\n".join(lines) + "\n")
    db = {}
    if os.path.exists(a.traffic_json):
        db = json.load(open(a.traffic_json))
    db[f"{a.workload}/{a.path}"] = {"library_build": a.build,
                                     "hbm_bytes_per_launch": round(sum(traffic.values())),
                                     "per_kernel_bytes": {k[:90]: round(v) for k, v in traffic.items()},
                                     "summary": os.path.basename(a.out)}
    write_atomic(a.traffic_json, json.dumps(db, indent=1))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
