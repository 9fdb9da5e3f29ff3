"""Benchmark of the fused rank-sum + residual-add + RMSNorm epilogue on one MI355X.

One step = one arrms_fused call over the headline workload (R=4 rank inputs,
1024 x 6144 bf16 rows, per-row input scales, plain RMSNorm, bf16 output),
with its inputs already resident in HBM. The timed calls cycle through enough
rotating buffer sets (>= 512 MiB in total, twice the 256 MB Infinity Cache) that
every call reads cold data from HBM. Calls are captured in a HIP graph and
timed with HIP events on the stream the kernels run on.

Prints one JSON line:
  value       achieved GB/s by the metric's byte count (R+2)*M*H*2 + H*2
  roofline    algorithmic bytes per launch ((R+3)*M*H*e + H*e: R inputs and the
              residual read, out and residual_out written, the weight) over the
              measured kernel duration, against MI355X's 8 TB/s HBM peak
  cpu_baseline  the CPU oracle, single-threaded, on the same workload
  quant_epilogues  per-token FP8, per-group FP8 and MXFP4 outputs on the FP8
              workload's rows (R=4, 2800 x 6144 fp16, gemma_norm)
  allreduce_sum the plain rank all-reduce (no norm) over a message of the same
              rank inputs' size (4 x 1024 x 6144 bf16), with its own roofline
              fraction; --sum-only prints that measurement as the line instead
  copy_reference a plain 256 MiB device-to-device copy on the same GPU (read
              plus written bytes per second), for context
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak) for fused sum+RMSNorm, R=4, H=6144"
PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=4096,
                   help="untimed calls first: the per-call time keeps falling over the first ~500 "
                        "calls (clocks and memory settling), so warm up well past that")
    p.add_argument("--workload", default="r4_m1024_h6144_bf16_rowscale")
    p.add_argument("--path", choices=("auto", "one", "two"), default="auto")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="bound on the CPU-baseline work")
    p.add_argument("--no-other-path", action="store_true", help="time only the chosen path")
    p.add_argument("--no-hot", action="store_true", help="skip the cache-resident context number")
    p.add_argument("--no-sum", action="store_true",
                   help="skip the plain rank all-reduce (no norm) timing")
    p.add_argument("--no-strided", action="store_true", help="skip the padded-rows timing")
    p.add_argument("--no-copy-reference", action="store_true",
                   help="skip the plain 256 MiB device copy timed for reference")
    p.add_argument("--no-quant", action="store_true",
                   help="skip the per-token / per-group FP8 / MXFP4 epilogue timings")
    p.add_argument("--replays", type=int, default=20,
                   help="further timed replays of the chosen path, for median/min (0: none)")
    p.add_argument("--sum-only", action="store_true",
                   help="time only the plain rank all-reduce (R=4, 1024 x 6144 bf16 message)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 256 MiB device-to-device copy (4 times) so that a "
                        "profiler's FETCH_SIZE/WRITE_SIZE can be scaled by a kernel of known size")
    return p.parse_args()


def sources_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "all_reduce_residual_rank_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, path: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were
    taken on the current kernel sources; else None."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(f):
        return None
    try:
        d = json.load(open(f))
    except (OSError, ValueError):
        return None
    e = d.get(f"{workload}/{path}")
    if not e or e.get("sources_digest") != digest:
        return None
    return e.get("hbm_bytes_per_launch")


class Sets:
    """Rotating device buffer sets of one workload."""

    def __init__(self, wl, nsets, torch):
        from all_reduce_residual_rank_amd import workloads as wlmod
        dev = torch.device("cuda")
        T = wlmod.DTYPES[wl.dtype]
        xs, res, w = wlmod.make_inputs(wl, seed=0)
        self.sets = []
        for s in range(nsets):
            d = {"xs": [x.to(dev) for x in xs], "res": res.to(dev), "w": w.to(dev),
                 "rout": torch.empty(wl.M, wl.H, dtype=T, device=dev),
                 "out": torch.empty(wl.M, wl.H, dtype=T, device=dev) if (wl.mirror or not wl.fp8) else None,
                 "q": torch.empty(wl.M, wl.H, dtype=torch.uint8, device=dev) if wl.fp8 else None,
                 "sc": torch.empty(wl.M, dtype=torch.float32, device=dev) if wl.fp8 else None}
            self.sets.append(d)


def call(arrms, wl, d, flags, stream):
    arrms.arrms_fused(d["xs"], d["res"], d["w"], d["out"], d["rout"], d["q"], d["sc"], eps=wl.eps,
                      flags=flags, M=wl.M, H=wl.H, stream=stream)


def time_graph(torch, calls, steps, warmup, extra=None):
    """Warm up, then time exactly `steps` calls replayed from one HIP graph.
    calls: functions f(stream) that each enqueue one call; used in turn.
    extra: a list that receives the ms of further timed replays (len(extra)
    given as a count in extra[0]), for the spread; the first timing is the
    one returned."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    n = len(calls)
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk, stream=s):
        for i in range(steps):
            calls[i % n](s)
    torch.cuda.synchronize()
    if warmup > 0 and warmup % steps == 0:
        # warm up with the timed graph itself (its first replays also carry the
        # graph's one-time upload)
        with torch.cuda.stream(s):
            for _ in range(warmup // steps):
                gk.replay()
    elif warmup > 0:
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=s):
            for i in range(warmup):
                calls[i % n](s)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            gw.replay()
        del gw
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        gk.replay()
        e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    if extra:
        n = int(extra.pop())
        for _ in range(n):
            with torch.cuda.stream(s):
                e0.record(s)
                gk.replay()
                e1.record(s)
            torch.cuda.synchronize()
            extra.append(e0.elapsed_time(e1))
    del gk
    return ms


def time_path(torch, arrms, wl, sets, flags, steps, warmup, extra=None):
    calls = [lambda st, d=d: call(arrms, wl, d, flags, st) for d in sets.sets]
    return time_graph(torch, calls, steps, warmup, extra)


def copy_reference(torch, nbytes=256 << 20, reps=10):
    """A plain device-to-device copy (torch's copy_) of nbytes on this GPU, as a
    reference for what a simple one-stream streaming kernel reaches here: GB/s
    counting the bytes read and the bytes written."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    del src, dst
    return {"kind": "torch copy_ device to device", "bytes_per_copy": 2 * nbytes, "us_per_copy": round(us, 2),
            "achieved": round(2 * nbytes / (us * 1e-6) / 1e9, 1), "unit": "GB/s"}


def time_strided(torch, arrms, wl, pad, steps, warmup):
    """The workload through arrms_fused_strided: every matrix a column window
    of an [M][H + pad] allocation (row stride H + pad elements)."""
    from all_reduce_residual_rank_amd import workloads as wlmod
    dev = torch.device("cuda")
    T = wlmod.DTYPES[wl.dtype]
    xs, res, w = wlmod.make_inputs(wl, seed=0)
    ld = wl.H + pad

    def win(src=None):
        base = torch.empty(wl.M, ld, dtype=T, device=dev)
        v = base[:, :wl.H]
        if src is not None:
            v.copy_(src)
        return v

    nsets = max(2, -(-ROTATE_BYTES // ((wl.R + 3) * wl.M * ld * wl.esize)))
    sets = [{"xs": [win(x) for x in xs], "res": win(res), "w": w.to(dev), "out": win(), "rout": win()}
            for _ in range(nsets)]

    def one(d, st):
        arrms.arrms_fused_strided(d["xs"], d["res"], d["w"], d["out"], d["rout"], eps=wl.eps,
                                  flags=wl.flags | arrms.FORCE_ONE_STAGE, stream=st)

    calls = [lambda st, d=d: one(d, st) for d in sets]
    ms = time_graph(torch, calls, steps, warmup)
    del sets
    return ms * 1000.0 / steps


def time_quant(torch, arrms, wl, quant, steps, warmup):
    """The workload with a quantised output through arrms_fused_quant (no T
    mirror). Returns (us per call, algorithmic bytes per call)."""
    from all_reduce_residual_rank_amd import workloads as wlmod
    dev = torch.device("cuda")
    T = wlmod.DTYPES[wl.dtype]
    e = wl.esize
    M, H = wl.M, wl.H
    if quant == arrms.QUANT_FP8_TOKEN:
        qbytes, sbytes = M * H, M * 4
    elif quant == arrms.QUANT_FP8_GROUP:
        qbytes, sbytes = M * H, M * (H // arrms.FP8_GROUP_SIZE) * 4
    else:
        qbytes, sbytes = M * H // 2, M * (H // arrms.MX_BLOCK)
    algo = (wl.R + 2) * M * H * e + H * e + qbytes + sbytes
    xs, res, w = wlmod.make_inputs(wl, seed=0)
    nsets = max(2, -(-ROTATE_BYTES // algo))
    sets = [{"xs": [x.to(dev) for x in xs], "res": res.to(dev), "w": w.to(dev),
             "rout": torch.empty(M, H, dtype=T, device=dev),
             "q": torch.empty(qbytes, dtype=torch.uint8, device=dev),
             "s": torch.empty(sbytes, dtype=torch.uint8, device=dev)} for _ in range(nsets)]
    flags = (wl.flags & ~arrms.FP8) | arrms.FORCE_ONE_STAGE

    def one(d, st):
        arrms.arrms_fused_quant(d["xs"], d["res"], d["w"], None, d["rout"], d["q"], d["s"], eps=wl.eps,
                                flags=flags, quant=quant, M=M, H=H, stream=st)

    ms = time_graph(torch, [lambda st, d=d: one(d, st) for d in sets], steps, warmup)
    del sets
    return ms * 1000.0 / steps, algo


def time_sum(torch, arrms, case, R, steps, warmup):
    """The plain rank all-reduce on one message over rotating buffer sets.
    Returns (us per call, algorithmic bytes per call)."""
    from all_reduce_residual_rank_amd import workloads as wlmod
    dev = torch.device("cuda")
    xs = wlmod.make_sum_inputs(R, case.numel, 0, case.dtype)
    nsets = max(2, -(-ROTATE_BYTES // ((R + 1) * case.nbytes)))
    sets = [([x.to(dev) for x in xs], torch.empty(case.numel, dtype=wlmod.DTYPES[case.dtype], device=dev))
            for _ in range(nsets)]
    flags = wlmod.DT_CODE[case.dtype]
    calls = [lambda st, d=d: arrms.arrms_allreduce_sum(d[0], d[1], flags=flags, stream=st) for d in sets]
    ms = time_graph(torch, calls, steps, warmup)
    del sets
    return ms * 1000.0 / steps, (R + 1) * case.nbytes


def time_hot(torch, arrms, wl, sets, flags, reps=64):
    """Single buffer set replayed: cache-resident ("hot") context number."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            call(arrms, wl, sets.sets[0], flags, s)
    torch.cuda.synchronize()
    res = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1000.0 / reps)
    return min(res)


def read_clocks(torch):
    """Current shader and memory clocks of device 0, read from the amdgpu
    driver's sysfs DPM tables (the entry marked with '*'); None where the files
    are not readable. A file read, so nothing is spawned from this process."""
    try:
        p = torch.cuda.get_device_properties(0)
        root = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    except (AttributeError, RuntimeError):
        return None
    out = {}
    for key, name in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk")):
        try:
            with open(os.path.join(root, name)) as f:
                cur = [ln.split(":", 1)[1].replace("*", "").strip() for ln in f if ln.rstrip().endswith("*")]
        except (OSError, IndexError):
            continue
        if cur:
            out[key] = cur[0]
    return out or None


def cpu_baseline(wl, budget_s):
    """The oracle as it stands, single-threaded, on row samples of the workload."""
    import numpy as np
    import torch
    import oracle
    from all_reduce_residual_rank_amd import workloads as wlmod

    xs, res, w = wlmod.make_inputs(wl, seed=0)

    def bits(t):
        if t.dtype == torch.float32:
            return t.numpy()
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    xb = [bits(x) for x in xs]
    rb, wb = bits(res), bits(w)
    def once(n):
        t0 = time.perf_counter()
        oracle.fused(xb, rb, wb, wl.eps, wl.flags & 0xF, rows=(0, n))
        return time.perf_counter() - t0

    probe = min(wl.M, 8)
    t_probe = once(probe)
    rows = max(1, min(wl.M, int(probe * (budget_s / 3.0) / max(t_probe, 1e-9))))
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (len(times) < 15 and time.perf_counter() - t_start < budget_s):
        times.append(once(rows))
    t = statistics.median(times)
    e = wl.esize
    metric_bytes = (wl.R + 2) * rows * wl.H * e + wl.H * e
    out = {"value": round(metric_bytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"rows 0..{rows - 1} of the workload ({rows}x{wl.H}, R={wl.R}), "
                     f"median of {len(times)} runs, {t * 1e3:.1f} ms each",
           "us_per_row": round(t / rows * 1e6, 3)}
    # the same sample split by rows over the host's cores (the oracle's C code
    # runs outside the GIL), for context
    from concurrent.futures import ThreadPoolExecutor
    n = max(1, min(len(os.sched_getaffinity(0)), 16, rows))
    bounds = [(rows * i // n, rows * (i + 1) // n) for i in range(n)]

    def part(b):
        oracle.fused(xb, rb, wb, wl.eps, wl.flags & 0xF, rows=b)

    with ThreadPoolExecutor(n) as ex:
        tt = []
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(part, bounds))
            tt.append(time.perf_counter() - t0)
    tm = statistics.median(tt)
    out["threads"] = {"value": round(metric_bytes / tm / 1e9, 4), "cores": n,
                      "sample": f"the same rows split over {n} threads, median of 3 runs, {tm * 1e3:.1f} ms each"}
    out["cpu_model"] = cpu_model()
    return out


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU's share of the collective; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from all_reduce_residual_rank_amd import arrms
    from all_reduce_residual_rank_amd import workloads as wlmod

    wl = wlmod.BY_NAME[args.workload]
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.sum_only:
        case = wlmod.SUM_HEADLINE
        us, nbytes = time_sum(torch, arrms, case, 4, args.steps, args.warmup)
        gbs = nbytes / (us * 1e-6) / 1e9
        digest = sources_digest()
        print(json.dumps({
            "metric": "µs/call and achieved HBM GB/s of the plain rank all-reduce, R=4",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(us / 1000.0, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": case.dtype, "data": "synthetic",
            "config": {"workload": case.name, "R": 4, "numel": case.numel},
            "us_per_call": round(us, 3),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_GBS, 4),
                         "traffic": load_traffic(case.name, "flat", digest),
                         "algorithmic_bytes": nbytes, "kernel": "flat_kernel"},
            "sources_digest": digest}), flush=True)
        return
    e = wl.esize
    set_bytes = (wl.R + 3) * wl.M * wl.H * e
    nsets = max(2, -(-ROTATE_BYTES // set_bytes))
    sets = Sets(wl, nsets, torch)
    arrms.arrms_reserve_staging(0)

    path_flags = {"one": arrms.FORCE_ONE_STAGE, "two": arrms.FORCE_TWO_STAGE, "auto": 0}
    auto_path = {arrms.PATH_ONE_STAGE: "one", arrms.PATH_TWO_STAGE: "two"}[
        arrms.arrms_query_path(wl.M, wl.H, wl.R, wl.flags)]
    chosen = auto_path if args.path == "auto" else args.path
    reps = [float(args.replays)]
    ms = time_path(torch, arrms, wl, sets, wl.flags | path_flags[chosen], args.steps, args.warmup, reps)
    us = ms * 1000.0 / args.steps
    rep_us = sorted(r * 1000.0 / args.steps for r in reps)
    metric_bytes = (wl.R + 2) * wl.M * wl.H * e + wl.H * e
    algo_bytes = (wl.R + 3) * wl.M * wl.H * e + wl.H * e
    if wl.fp8:
        algo_bytes = (wl.R + 1) * wl.M * wl.H * e + wl.H * e + wl.M * wl.H + wl.M * 4 + \
            (wl.M * wl.H * e if wl.mirror else 0) + wl.M * wl.H * e
    gbs = metric_bytes / (us * 1e-6) / 1e9
    achieved = algo_bytes / (us * 1e-6) / 1e9

    other = {}
    for p in ("one", "two"):
        if p == chosen:
            other[p] = round(us, 3)
        elif not args.no_other_path:
            ms2 = time_path(torch, arrms, wl, sets, wl.flags | path_flags[p], args.steps, args.warmup)
            other[p] = round(ms2 * 1000.0 / args.steps, 3)
    hot = None if args.no_hot else time_hot(torch, arrms, wl, sets, wl.flags | path_flags[chosen])
    digest = sources_digest()
    traffic = load_traffic(wl.name, chosen, digest)

    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "R": wl.R, "M": wl.M, "H": wl.H, "dtype": wl.dtype,
                   "gemma": wl.gemma, "fp8": wl.fp8, "path": chosen, "rotating_sets": nsets,
                   "compute": "fp32 rank sums, fp64 row statistics"},
        "us_per_call": round(us, 3), "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
        "metric_bytes": metric_bytes,
        "path_us": other, "hot_us_cache_resident": None if hot is None else round(hot, 3),
        "replays": None if not rep_us else {"n": len(rep_us), "median_us": round(statistics.median(rep_us), 3),
                                             "min_us": round(rep_us[0], 3), "max_us": round(rep_us[-1], 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": algo_bytes,
                     "kernel": "row_kernel" if chosen == "one" else "flat_kernel+row_kernel"},
        "sources_digest": digest,
        "device": torch.cuda.get_device_name(0),
        "arch": torch.cuda.get_device_properties(0).gcnArchName,
    }
    if not args.no_sum:
        # the plain rank all-reduce (no norm) on the same rank inputs' size
        case = wlmod.SUM_HEADLINE
        sum_us, sum_bytes = time_sum(torch, arrms, case, 4, args.steps, args.warmup)
        line["allreduce_sum"] = {"message": case.name, "R": 4, "us_per_call": round(sum_us, 3),
                                 "achieved": round(sum_bytes / (sum_us * 1e-6) / 1e9, 2),
                                 "unit": "GB/s", "algorithmic_bytes": sum_bytes,
                                 "frac": round(sum_bytes / (sum_us * 1e-6) / 1e9 / PEAK_GBS, 4),
                                 "kernel": "flat_kernel"}
    if not args.no_strided and not wl.fp8:
        # padded rows (row stride H + 64 elements) through arrms_fused_strided
        st_us = time_strided(torch, arrms, wl, 64, args.steps, args.warmup)
        line["strided"] = {"row_stride": wl.H + 64, "us_per_call": round(st_us, 3),
                           "achieved": round(algo_bytes / (st_us * 1e-6) / 1e9, 2), "unit": "GB/s",
                           "frac": round(algo_bytes / (st_us * 1e-6) / 1e9 / PEAK_GBS, 4),
                           "kernel": "row_kernel"}
    if not args.no_quant:
        # the quant forms of the epilogue on the FP8 workload's rows (R=4,
        # 2800 x 6144 fp16, gemma_norm, no T mirror)
        qwl = wlmod.FP8_GEMMA
        qres = {}
        for name, qm in (("per_token_fp8", arrms.QUANT_FP8_TOKEN), ("per_group_fp8", arrms.QUANT_FP8_GROUP),
                         ("mxfp4", arrms.QUANT_MXFP4)):
            q_us, q_bytes = time_quant(torch, arrms, qwl, qm, args.steps, args.warmup)
            qres[name] = {"us_per_call": round(q_us, 3), "algorithmic_bytes": q_bytes,
                          "achieved": round(q_bytes / (q_us * 1e-6) / 1e9, 2),
                          "frac": round(q_bytes / (q_us * 1e-6) / 1e9 / PEAK_GBS, 4)}
        line["quant_epilogues"] = {"workload": qwl.name, "unit": "GB/s", "kernel": "row_kernel", **qres}
    if not args.no_copy_reference and not args.calibrate_copy:
        # (not in profiling runs: their counters are scaled by the one calibration copy)
        line["copy_reference"] = copy_reference(torch)
    clocks = read_clocks(torch)
    if clocks:
        line["clocks"] = clocks
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
