"""Benchmark of the fused rank-sum + residual-add + RMSNorm epilogue on one MI355X.

One step = one arrms_fused call over the headline workload (R=4 rank inputs,
1024 x 6144 bf16 rows, per-row input scales, plain RMSNorm, bf16 output),
with its inputs already resident in HBM. The timed calls cycle through enough
rotating buffer sets (>= 512 MiB in total, twice the 256 MB Infinity Cache) that
every call reads cold data from HBM. Calls are timed with HIP events on the
stream the kernels run on, as the protocol below describes.

Timing protocol (every figure below):
  pre-roll    the timed graph itself is replayed, untimed, until at least
              PREROLL_CALLS calls and PREROLL_SECONDS have run: the per-call time
              of a fresh process keeps falling over its first few hundred calls
              while clocks and memory settle (reported as preroll_calls);
  warm-up     then --warmup further calls, untimed;
  timed       exactly --steps calls of the entry point, eager, on one stream,
              between two HIP events. Each block of timed calls is queued behind
              untimed filler on the same stream (replays of a graph of the same
              calls, then LEAD_IN_CALLS eager calls), long enough that the host
              has issued the whole block before the GPU reaches its first event:
              the figure is the GPU time of back-to-back calls, with no host
              launch gap and no per-graph launch cost inside. Every block starts
              at the first buffer set. Further blocks, each queued the same way
              after the previous one has finished, give the spread (replays). This is the headline's own measurement; every
              other figure (other workloads and paths, the quant forms, the sum,
              the probe, the sweep) is the us per call inside graphs of at least
              64 calls replayed back to back (time_graph_calls), because the
              host's cost per eager call (tens of us) would outrun the GPU's for
              small launches; graph_us_per_call gives the headline that way too.

Prints one JSON line:
  value       achieved GB/s by the metric's byte count (R+2)*M*H*2 + H*2
  roofline    algorithmic bytes per launch ((R+3)*M*H*e + H*e: R inputs and the
              residual read, out and residual_out written, the weight) over the
              measured kernel duration, against MI355X's 8 TB/s HBM peak
  probe       a data-movement-only kernel over the same bytes (5 read and 2 write
              streams per row, no arithmetic), the measured ceiling the fused
              kernel is compared with (frac_of_probe); with its read side and
              its write side timed alone on the same buffers
  workloads   every workload of the scope table (the 16-row decode case, the
              headline on both paths, the FP8 workload, the R=8 wide rows on both
              paths, the tail/decode sweep) with us/call per path
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
import ctypes
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
PREROLL_CALLS = 4096
PREROLL_SECONDS = 0.5
LEAD_IN_CALLS = 4            # untimed eager calls between the filler and each timed block
CALIBRATE_BYTES = 256 << 20  # read and written by each calibration dispatch (--calibrate-copy)
MAX_TIMED_CALLS = 4096       # small workloads: more timed calls, so that more distinct data is touched
BANDWIDTH_BOUND_BYTES = 32 << 20   # per call: below this a launch is latency-bound (report us only)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=256,
                   help="untimed calls after the pre-roll (which always runs first)")
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
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the other workloads of the scope table")
    p.add_argument("--no-probe", action="store_true", help="skip the data-movement probe")
    p.add_argument("--replays", type=int, default=20,
                   help="further timed replays of the chosen path, for median/min (0: none)")
    p.add_argument("--sum-only", action="store_true",
                   help="time only the plain rank all-reduce (R=4, 1024 x 6144 bf16 message)")
    p.add_argument("--probe-only", action="store_true",
                   help="time only the data-movement probe of the chosen workload")
    p.add_argument("--sweep", action="store_true",
                   help="time every launch shape, load window and path of the row kernel over a grid of "
                        "rows x hidden x ranks (bf16 T output, fp16 gemma per-token FP8) and write a CSV")
    p.add_argument("--sweep-out", default=os.path.join(ROOT, "profiles", "dispatch_sweep.csv"))
    p.add_argument("--sweep-m", default="1,16,64,256,512,1024,2048,2800,4096")
    p.add_argument("--sweep-h", default="512,2880,4096,6144,7168,8192")
    p.add_argument("--sweep-r", default="2,4,8")
    p.add_argument("--sweep-kinds", default="bf16,fp16_fp8")
    p.add_argument("--graph", action="store_true",
                   help="time the chosen workload inside graphs of --steps calls replayed back to back "
                        "(as every figure but the headline is), e.g. for kernel traces of latency-bound launches")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run 4 dispatches of the probe kernel that each read and write 256 MiB, so "
                        "that a profiler's FETCH_SIZE/WRITE_SIZE can be scaled by a kernel of known traffic")
    return p.parse_args()


def sources_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "all_reduce_residual_rank_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        path = os.path.join(csrc, name)
        if not os.path.isfile(path):  # e.g. a Python cache directory
            continue
        with open(path, "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def file_sha256(path: str) -> str | None:
    try:
        with open(path, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None


def rocm_version() -> str | None:
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def library_build() -> str | None:
    """The build of libarrms.so the run loads: the first 16 hex digits of its
    SHA-256. Committed counter traffic is keyed on it (a change of comments or
    of anything that leaves the library's bytes alone keeps the key)."""
    from all_reduce_residual_rank_amd import arrms
    h = file_sha256(arrms.LIB_PATH)
    return h[:16] if h else None


def load_traffic(workload: str, path: str, build: str | None):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were
    taken on this build of the library; else None."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(f):
        return None
    try:
        d = json.load(open(f))
    except (OSError, ValueError):
        return None
    e = d.get(f"{workload}/{path}")
    if not e or not build or e.get("library_build") != build:
        return None
    return e.get("hbm_bytes_per_launch")


# ---- timing ----------------------------------------------------------------

class Graph:
    """`ncalls` calls (cycling through `calls`) captured in one HIP graph on a
    side stream: the pre-roll, and the untimed filler that keeps the GPU busy
    while the host queues the timed calls."""

    def __init__(self, torch, calls, ncalls, stream):
        self.torch = torch
        self.ncalls = ncalls
        self.s = stream
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g, stream=self.s):
            for i in range(ncalls):
                calls[i % len(calls)](self.s)
        torch.cuda.synchronize()
        self.gpu_s = None  # GPU time of one replay

    def replay(self, n=1):
        with self.torch.cuda.stream(self.s):
            for _ in range(n):
                self.g.replay()

    def preroll(self, min_calls=PREROLL_CALLS, min_seconds=PREROLL_SECONDS):
        """Untimed replays until at least min_calls calls and min_seconds have run;
        returns the number of calls. Also times one replay on the GPU."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        done = 0
        batch = max(1, 256 // self.ncalls)
        while done < min_calls or time.perf_counter() - t0 < min_seconds:
            self.replay(batch)
            done += batch * self.ncalls
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.s):
            e0.record(self.s)
            self.g.replay()
            e1.record(self.s)
        torch.cuda.synchronize()
        self.gpu_s = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
        return done + self.ncalls


def time_calls(torch, calls, steps, warmup, replays=0, ncalls=None, preroll=(PREROLL_CALLS, PREROLL_SECONDS)):
    """Pre-roll, warm up, then time exactly `ncalls` (default `steps`) calls, and
    `replays` further blocks of as many calls, each block between two HIP events.

    The timed calls are ordinary eager calls of the entry point on one stream.
    Before each block the stream gets untimed filler -- replays of a graph of
    the same calls, then a few eager calls -- long enough (twice the host's
    time to issue them and the block) that the host has queued the whole block
    before the GPU reaches its first event: the events see back-to-back
    execution only, with no host launch gap and no per-graph launch cost
    inside. Each block starts at the first of `calls` and is queued once the
    previous one has finished. Returns us per call of the first block, the
    spread of the others and the pre-roll count."""
    ncalls = steps if ncalls is None else ncalls
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = Graph(torch, calls, min(max(ncalls, 64), 512), s)
    pre = g.preroll(*preroll)
    # warm-up: eager calls, whose host time per call sizes the filler
    host = []
    for i in range(max(warmup, 16)):
        h0 = time.perf_counter()
        calls[i % len(calls)](s)
        host.append(time.perf_counter() - h0)
        if i % 64 == 63:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    h_call = statistics.median(host)
    lead = min(LEAD_IN_CALLS, len(calls))
    nfill = max(1, -(-int((2.0 * (ncalls + lead) * h_call + 200e-6) * 1e6) // int(g.gpu_s * 1e6)))
    us = []
    with torch.cuda.stream(s):
        for b in range(1 + replays):
            # filler, then a few untimed eager calls (the first eager launches
            # after a graph replay are not yet back to back), then the block.
            # Every block starts at the first buffer set, so all blocks read the
            # same mix of sets, and the device is synchronised after each block,
            # so the host queues each block against an empty queue.
            g.replay(nfill)
            for i in range(lead):
                calls[(len(calls) - lead + i) % len(calls)](s)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for i in range(ncalls):
                calls[i % len(calls)](s)
            e1.record(s)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1000.0 / ncalls)
    out = {"us_per_call": us[0], "preroll_calls": pre, "warmup_calls": max(warmup, 16), "calls_per_block": ncalls,
           "host_us_per_call": round(h_call * 1e6, 1), "filler_calls": nfill * g.ncalls}
    if replays:
        r = sorted(us[1:])
        out["replays"] = {"n": len(r), "median_us": round(statistics.median(r), 3), "min_us": round(r[0], 3),
                          "max_us": round(r[-1], 3)}
    del g
    return out


def time_graph_calls(torch, calls, ncalls, nrep=5, preroll=(PREROLL_CALLS, PREROLL_SECONDS)):
    """us per call inside HIP graphs: a graph of `ncalls` calls (cycling through
    `calls`) is pre-rolled, then replayed nrep times back to back with a HIP
    event after each replay; returns the median and the least us per call over
    the replays. For everything but the headline: graphs keep the host's cost
    per call (tens of us through Python) out of the GPU's way even for calls of
    a few microseconds, and a graph of many calls amortises the graph's own
    launch cost."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = Graph(torch, calls, ncalls, s)
    g.preroll(*preroll)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nrep + 1)]
    with torch.cuda.stream(s):
        g.g.replay()  # lead-in, untimed
        ev[0].record(s)
        for i in range(nrep):
            g.g.replay()
            ev[i + 1].record(s)
    torch.cuda.synchronize()
    us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1000.0 / ncalls for i in range(nrep))
    del g
    return statistics.median(us), us[0]


# ---- workloads ------------------------------------------------------------

class Sets:
    """Rotating device buffer sets of one workload (nsets copies of its inputs,
    made on the device from one upload)."""

    def __init__(self, wl, nsets, torch):
        from all_reduce_residual_rank_amd import workloads as wlmod
        dev = torch.device("cuda")
        T = wlmod.DTYPES[wl.dtype]
        xs, res, w = wlmod.make_inputs(wl, seed=0)
        xd = [x.to(dev) for x in xs]
        rd, wd = res.to(dev), w.to(dev)
        self.sets = []
        for s in range(nsets):
            d = {"xs": [x.clone() for x in xd], "res": rd.clone(), "w": wd,
                 "rout": torch.empty(wl.M, wl.H, dtype=T, device=dev),
                 "out": torch.empty(wl.M, wl.H, dtype=T, device=dev) if (wl.mirror or not wl.fp8) else None,
                 "q": torch.empty(wl.M, wl.H, dtype=torch.uint8, device=dev) if wl.fp8 else None,
                 "sc": torch.empty(wl.M, dtype=torch.float32, device=dev) if wl.fp8 else None}
            self.sets.append(d)


def call(arrms, wl, d, flags, stream):
    arrms.arrms_fused(d["xs"], d["res"], d["w"], d["out"], d["rout"], d["q"], d["sc"], eps=wl.eps,
                      flags=flags, M=wl.M, H=wl.H, stream=stream)


def algo_bytes_of(wl) -> int:
    """Bytes one call must move: the R inputs and the residual read, residual_out
    and the T output (or FP8 codes + scales, plus the optional mirror) written,
    and the weight."""
    e = wl.esize
    n = wl.M * wl.H
    if wl.fp8:
        return (wl.R + 2) * n * e + wl.H * e + n + wl.M * 4 + (n * e if wl.mirror else 0)
    return (wl.R + 3) * n * e + wl.H * e


def metric_bytes_of(wl) -> int:
    return (wl.R + 2) * wl.M * wl.H * wl.esize + wl.H * wl.esize


def nsets_for(wl, ncalls) -> int:
    set_bytes = (wl.R + 3) * wl.M * wl.H * wl.esize
    return max(2, min(ncalls, -(-ROTATE_BYTES // set_bytes)))


def calls_for(wl, steps) -> int:
    """Timed calls for a workload timed beside the headline: at least `steps`,
    and for small workloads enough to touch ROTATE_BYTES of distinct data (capped)."""
    set_bytes = (wl.R + 3) * wl.M * wl.H * wl.esize
    return max(steps, min(MAX_TIMED_CALLS, -(-ROTATE_BYTES // set_bytes)))


def time_workload(torch, arrms, wl, paths, steps, warmup, sets=None):
    """us/call of a workload on each of `paths` over rotating buffer sets, inside
    graphs (time_graph_calls)."""
    ncalls = calls_for(wl, steps)
    own = sets is None
    if own:
        sets = Sets(wl, nsets_for(wl, ncalls), torch)
    res = {"R": wl.R, "M": wl.M, "H": wl.H, "dtype": wl.dtype, "gemma": wl.gemma, "fp8": wl.fp8,
           "calls_per_graph": ncalls,
           "footprint_bytes": min(ncalls, len(sets.sets)) * algo_bytes_of(wl),
           "metric_bytes": metric_bytes_of(wl), "algorithmic_bytes": algo_bytes_of(wl)}
    bw = algo_bytes_of(wl) >= BANDWIDTH_BOUND_BYTES
    pf = {"one": arrms.FORCE_ONE_STAGE, "two": arrms.FORCE_TWO_STAGE}
    for p in paths:
        calls = [lambda st, d=d: call(arrms, wl, d, wl.flags | pf[p], st) for d in sets.sets]
        us, us_min = time_graph_calls(torch, calls, ncalls, preroll=(PREROLL_CALLS, 0.2))
        r = {"us_per_call": round(us, 3), "min_us": round(us_min, 3)}
        if bw:
            r["metric_gbs"] = round(metric_bytes_of(wl) / (us * 1e-6) / 1e9, 1)
            r["achieved_gbs"] = round(algo_bytes_of(wl) / (us * 1e-6) / 1e9, 1)
            r["frac"] = round(algo_bytes_of(wl) / (us * 1e-6) / 1e9 / PEAK_GBS, 4)
        res[p] = r
    res["bound"] = "hbm" if bw else "latency"
    if own:
        del sets
        torch.cuda.empty_cache()
    return res


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
    us, _ = time_graph_calls(torch, calls, max(steps, 64))
    del sets
    return us


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
    xd = [x.to(dev) for x in xs]
    rd = res.to(dev)
    sets = [{"xs": [x.clone() for x in xd], "res": rd.clone(), "w": w.to(dev),
             "rout": torch.empty(M, H, dtype=T, device=dev),
             "q": torch.empty(qbytes, dtype=torch.uint8, device=dev),
             "s": torch.empty(sbytes, dtype=torch.uint8, device=dev)} for _ in range(nsets)]
    flags = (wl.flags & ~arrms.FP8) | arrms.FORCE_ONE_STAGE

    def one(d, st):
        arrms.arrms_fused_quant(d["xs"], d["res"], d["w"], None, d["rout"], d["q"], d["s"], eps=wl.eps,
                                flags=flags, quant=quant, M=M, H=H, stream=st)

    us, _ = time_graph_calls(torch, [lambda st, d=d: one(d, st) for d in sets], max(steps, 64))
    del sets
    return us, algo


def time_sum(torch, arrms, case, R, steps, warmup, standalone=False):
    """The plain rank all-reduce on one message over rotating buffer sets.
    Returns (us per call, algorithmic bytes per call): exactly `steps` eager calls
    when it is the line's own measurement (standalone), else inside graphs."""
    from all_reduce_residual_rank_amd import workloads as wlmod
    dev = torch.device("cuda")
    xs = wlmod.make_sum_inputs(R, case.numel, 0, case.dtype)
    nsets = max(2, -(-ROTATE_BYTES // ((R + 1) * case.nbytes)))
    xd = [x.to(dev) for x in xs]
    sets = [([x.clone() for x in xd], torch.empty(case.numel, dtype=wlmod.DTYPES[case.dtype], device=dev))
            for _ in range(nsets)]
    flags = wlmod.DT_CODE[case.dtype]
    calls = [lambda st, d=d: arrms.arrms_allreduce_sum(d[0], d[1], flags=flags, stream=st) for d in sets]
    if standalone:
        us = time_calls(torch, calls, steps, warmup)["us_per_call"]
    else:
        us, _ = time_graph_calls(torch, calls, max(steps, 64))
    del sets
    return us, (R + 1) * case.nbytes


def time_hot(torch, arrms, wl, sets, flags, reps=64):
    """Single buffer set, called again and again: cache-resident ("hot") context number."""
    _, us_min = time_graph_calls(torch, [lambda st: call(arrms, wl, sets.sets[0], flags, st)], reps,
                                 preroll=(reps * 8, 0.0))
    return us_min


# ---- the data-movement probe (measured ceiling) ---------------------------

def load_probe():
    """The streaming probe library (probe/libstream_probe.so), or None."""
    path = os.path.join(ROOT, "probe", "libstream_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.probe_rows.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(vp), ctypes.c_int,
                               ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.probe_rows.restype = ctypes.c_int
    lib.probe_rows_read.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_longlong, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.probe_rows_read.restype = ctypes.c_int
    lib.probe_rows_write.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, vp]
    lib.probe_rows_write.restype = ctypes.c_int
    return lib


def time_probe(torch, lib, wl, sets, steps, warmup, replays):
    """The probe over the workload's own rotating buffers: every row's R + 1 input
    streams read and two output streams written (residual_out and out), in the
    fused kernel's launch shape and load window, with no arithmetic; timed inside
    graphs (time_graph_calls). Also its two sides alone, each on the same
    buffers and launch shape: the reads with nothing written, the writes with
    nothing read."""
    from all_reduce_residual_rank_amd import arrms
    # the fused kernel's own launch shape and load window for this workload
    plan = arrms.arrms_query_launch(wl.M, wl.H, wl.R, wl.flags & ~arrms.FP8)
    ppt, tpr = plan["ppt"], plan["tpr"]
    window = {1: 2 if wl.R > 1 else 3, 2: 16, 3: 8}[plan["window"]]
    vp = ctypes.c_void_p

    def one(d, st):
        ins = (vp * (wl.R + 1))(*[x.data_ptr() for x in d["xs"]], d["res"].data_ptr())
        outs = (vp * 2)(d["rout"].data_ptr(), d["out"].data_ptr())
        rc = lib.probe_rows(ins, wl.R + 1, outs, 2, wl.M, wl.H * wl.esize, ppt, tpr, window, st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_rows failed: {rc}")

    sink = torch.zeros(max(wl.M, 1), dtype=torch.int32, device="cuda")

    def read(d, st):
        ins = (vp * (wl.R + 1))(*[x.data_ptr() for x in d["xs"]], d["res"].data_ptr())
        rc = lib.probe_rows_read(ins, wl.R + 1, sink.data_ptr(), wl.M, wl.H * wl.esize, ppt, tpr, window,
                                 st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_rows_read failed: {rc}")

    def write(d, st):
        outs = (vp * 2)(d["rout"].data_ptr(), d["out"].data_ptr())
        rc = lib.probe_rows_write(outs, 2, wl.M, wl.H * wl.esize, ppt, tpr, st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_rows_write failed: {rc}")

    n = max(steps, 64)
    us, us_min = time_graph_calls(torch, [lambda st, d=d: one(d, st) for d in sets.sets], n)
    rd_us, _ = time_graph_calls(torch, [lambda st, d=d: read(d, st) for d in sets.sets], n)
    wr_us, _ = time_graph_calls(torch, [lambda st, d=d: write(d, st) for d in sets.sets], n)
    del sink
    return {"us_per_call": us, "min_us": us_min, "read_only_us": rd_us, "write_only_us": wr_us,
            "launch": {"packs_per_thread": ppt, "threads_per_row": tpr, "load_window": window}}


# ---- launch-shape sweep ---------------------------------------------------

SWEEP_KINDS = {
    # name: (dtype, flags without the dtype, quant output, what)
    "bf16": ("bf16", 0, False, "bf16, plain weights, T output"),
    "fp16_fp8": ("fp16", 4 | 8, True, "fp16, gemma_norm, per-token FP8 without the T mirror"),
}
SWEEP_FIELDS = ("kind", "R", "M", "H", "variant", "path", "ppt", "tpr", "window", "us_median", "us_min",
                "calls_per_graph", "footprint_bytes", "auto_path", "auto_ppt", "auto_tpr", "auto_window",
                "auto_cap16", "blocks_per_cu", "cus")


def sweep(args):
    """Every valid one-stage launch shape (packs per thread 1-4, each load
    window), the two-stage path and the automatic choice, per point of the
    grid; median over 3 replays of a graph of n calls each (time_graph_calls,
    with a short pre-roll per variant after a long one for the process)."""
    import csv
    import math
    import torch
    from all_reduce_residual_rank_amd import arrms
    from all_reduce_residual_rank_amd import workloads as wlmod

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    arrms.arrms_reserve_staging(0)
    Ms = [int(x) for x in args.sweep_m.split(",")]
    Hs = [int(x) for x in args.sweep_h.split(",")]
    Rs = [int(x) for x in args.sweep_r.split(",")]
    kinds = args.sweep_kinds.split(",")
    os.makedirs(os.path.dirname(os.path.abspath(args.sweep_out)), exist_ok=True)
    # rows go to <out>.partial as they are measured (a run that is cut short
    # leaves what it has there) and the file takes its final name only when the
    # sweep is complete
    partial = args.sweep_out + ".partial"
    f = open(partial, "w", newline="")
    wr = csv.DictWriter(f, fieldnames=SWEEP_FIELDS)
    wr.writeheader()
    gen = torch.Generator(device=dev)
    warmed = False
    t_start = time.perf_counter()
    for kind in kinds:
        dtype, kflags, quant, _ = SWEEP_KINDS[kind]
        T = wlmod.DTYPES[dtype]
        e = 4 if dtype == "fp32" else 2
        base_flags = wlmod.DT_CODE[dtype] | kflags
        for R in Rs:
            for H in Hs:
                P = H * e // 16
                for M in Ms:
                    gen.manual_seed(M * 131 + H * 7 + R)
                    algo = (R + 2) * M * H * e + H * e + (M * H + M * 4 if quant else M * H * e)
                    est_us = max(3.0, algo / 5.5e12 * 1e6)
                    n = max(64, min(512, math.ceil(1000.0 / est_us)))
                    set_bytes = (R + 3) * M * H * e
                    nsets = max(2, min(n, -(-ROTATE_BYTES // set_bytes)))
                    sets = []
                    for _ in range(nsets):
                        d = {"xs": [torch.randn(M, H, generator=gen, device=dev).to(T) for _ in range(R)],
                             "res": torch.randn(M, H, generator=gen, device=dev).to(T),
                             "w": (torch.randn(H, generator=gen, device=dev) * 0.1).to(T),
                             "rout": torch.empty(M, H, dtype=T, device=dev),
                             "out": None if quant else torch.empty(M, H, dtype=T, device=dev),
                             "q": torch.empty(M, H, dtype=torch.uint8, device=dev) if quant else None,
                             "sc": torch.empty(M, dtype=torch.float32, device=dev) if quant else None}
                        sets.append(d)
                    auto = arrms.arrms_query_launch(M, H, R, base_flags)
                    variants = [("auto", 0, 0, 0, 0), ("two", arrms.FORCE_TWO_STAGE, 0, 0, 0)]
                    for ppt in (1, 2, 3, 4):
                        tpr = -(-P // ppt)
                        tpr = -(-tpr // 64) * 64
                        if tpr > (1024 if (ppt == 1 or dtype == "fp32") else 512):
                            continue
                        for win in (1, 2, 3):
                            if win == 3 and (R + 1) * ppt <= 8:
                                continue  # the medium window is the wide one for such rows
                            variants.append((f"ppt{ppt}_w{win}", arrms.FORCE_ONE_STAGE, ppt, tpr, win))
                    for name, force, ppt, tpr, win in variants:
                        def mk(d, force=force, ppt=ppt, win=win):
                            return lambda st: arrms.arrms_fused_config(
                                d["xs"], d["res"], d["w"], d["out"], d["rout"], d["q"], d["sc"], eps=1e-6,
                                flags=base_flags | force, ppt=ppt, load_window=win, M=M, H=H, stream=st)
                        calls = [mk(d) for d in sets]
                        pre = (PREROLL_CALLS, PREROLL_SECONDS) if not warmed else (n, 0.01)
                        warmed = True
                        med, least = time_graph_calls(torch, calls, n, nrep=3, preroll=pre)
                        if name == "auto":
                            path = "one" if auto["path"] == 1 else "two"
                            ppt_r, tpr_r, win_r = auto["ppt"], auto["tpr"], auto["window"]
                        elif name == "two":
                            path, ppt_r, tpr_r, win_r = "two", 0, 0, 0
                        else:
                            path, ppt_r, tpr_r, win_r = "one", ppt, tpr, win
                        wr.writerow({"kind": kind, "R": R, "M": M, "H": H, "variant": name, "path": path,
                                     "ppt": ppt_r, "tpr": tpr_r, "window": win_r,
                                     "us_median": round(med, 3), "us_min": round(least, 3),
                                     "calls_per_graph": n, "footprint_bytes": min(n, nsets) * set_bytes,
                                     "auto_path": auto["path"], "auto_ppt": auto["ppt"], "auto_tpr": auto["tpr"],
                                     "auto_window": auto["window"], "auto_cap16": auto["cap16"],
                                     "blocks_per_cu": auto["blocks_per_cu"], "cus": auto["cus"]})
                    f.flush()
                    print(f"sweep {kind} R={R} H={H} M={M}: {len(variants)} variants, "
                          f"{time.perf_counter() - t_start:.0f} s", flush=True)
                    del sets
                    torch.cuda.empty_cache()
    f.close()
    os.replace(partial, args.sweep_out)
    print(json.dumps({"sweep": args.sweep_out, "seconds": round(time.perf_counter() - t_start, 1)}), flush=True)


def calibrate(torch):
    """Four dispatches of the probe kernel (probe/libstream_probe.so), each
    reading CALIBRATE_BYTES and writing CALIBRATE_BYTES (two 128 MiB inputs, two
    128 MiB outputs): a kernel of known traffic, and the only probe dispatches of
    a profiled run, by which prof.py scales FETCH_SIZE and WRITE_SIZE to bytes."""
    lib = load_probe()
    if lib is None:
        raise SystemExit("--calibrate-copy needs probe/libstream_probe.so (python __graft_entry__.py)")
    n = CALIBRATE_BYTES // 2
    bufs = [torch.full((n,), 1, dtype=torch.uint8, device="cuda") for _ in range(4)]
    vp = ctypes.c_void_p
    ins = (vp * 2)(bufs[0].data_ptr(), bufs[1].data_ptr())
    outs = (vp * 2)(bufs[2].data_ptr(), bufs[3].data_ptr())
    row_bytes = 16384
    for _ in range(4):
        rc = lib.probe_rows(ins, 2, outs, 2, n // row_bytes, row_bytes, 2, 512, 16,
                            torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_rows failed: {rc}")
    torch.cuda.synchronize()
    del bufs


# ---- host facts -----------------------------------------------------------

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
    # runs outside the GIL), for context: every core of the process's affinity
    # mask, at most 16 (a host's CPU share for one GPU)
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
                      "affinity_cores": len(os.sched_getaffinity(0)),
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


def run_meta(torch, arrms):
    return {"rocm": rocm_version(), "torch_hip": getattr(torch.version, "hip", None),
            "libarrms_sha256": file_sha256(arrms.LIB_PATH), "sources_digest": sources_digest()}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU's share of the collective; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    import torch
    from all_reduce_residual_rank_amd import arrms
    from all_reduce_residual_rank_amd import workloads as wlmod

    wl = wlmod.BY_NAME[args.workload]
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate(torch)
    digest = sources_digest()
    build = library_build()
    if args.sum_only:
        case = wlmod.SUM_HEADLINE
        us, nbytes = time_sum(torch, arrms, case, 4, args.steps, args.warmup, standalone=True)
        gbs = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({
            "metric": "µs/call and achieved HBM GB/s of the plain rank all-reduce, R=4",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(us / 1000.0, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": case.dtype, "data": "synthetic",
            "config": {"workload": case.name, "R": 4, "numel": case.numel},
            "us_per_call": round(us, 3),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_GBS, 4),
                         "traffic": load_traffic(case.name, "flat", build),
                         "algorithmic_bytes": nbytes, "kernel": "flat_kernel"},
            "sources_digest": digest}), flush=True)
        return
    e = wl.esize
    ncalls = args.steps
    sets = Sets(wl, nsets_for(wl, ncalls), torch)
    if args.probe_only:
        lib = load_probe()
        if lib is None:
            raise SystemExit("probe/libstream_probe.so is not built (python __graft_entry__.py)")
        t = time_probe(torch, lib, wl, sets, args.steps, args.warmup, args.replays)
        print(json.dumps({"probe": wl.name, **t}), flush=True)
        return
    arrms.arrms_reserve_staging(0)

    path_flags = {"one": arrms.FORCE_ONE_STAGE, "two": arrms.FORCE_TWO_STAGE, "auto": 0}
    auto_path = {arrms.PATH_ONE_STAGE: "one", arrms.PATH_TWO_STAGE: "two"}[
        arrms.arrms_query_path(wl.M, wl.H, wl.R, wl.flags)]
    chosen = auto_path if args.path == "auto" else args.path
    calls = [lambda st, d=d: call(arrms, wl, d, wl.flags | path_flags[chosen], st) for d in sets.sets]
    if args.graph:
        gu, gmin = time_graph_calls(torch, calls, ncalls, nrep=max(3, args.replays))
        t = {"us_per_call": gu, "preroll_calls": PREROLL_CALLS, "warmup_calls": 0,
             "replays": {"n": max(3, args.replays), "median_us": round(gu, 3), "min_us": round(gmin, 3)}}
    else:
        t = time_calls(torch, calls, args.steps, args.warmup, replays=args.replays, ncalls=ncalls)
    us = t["us_per_call"]
    metric_bytes = metric_bytes_of(wl)
    algo_bytes = algo_bytes_of(wl)
    gbs = metric_bytes / (us * 1e-6) / 1e9
    achieved = algo_bytes / (us * 1e-6) / 1e9

    other = {}
    for p in ("one", "two"):
        if p == chosen:
            other[p] = round(us, 3)
        elif not args.no_other_path:
            c2 = [lambda st, d=d: call(arrms, wl, d, wl.flags | path_flags[p], st) for d in sets.sets]
            other[p] = round(time_calls(torch, c2, args.steps, args.warmup)["us_per_call"], 3)
    hot = None if args.no_hot else time_hot(torch, arrms, wl, sets, wl.flags | path_flags[chosen])
    traffic = load_traffic(wl.name, chosen, build)

    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "R": wl.R, "M": wl.M, "H": wl.H, "dtype": wl.dtype,
                   "gemma": wl.gemma, "fp8": wl.fp8, "path": chosen, "rotating_sets": len(sets.sets),
                   "compute": "fp32 rank sums, fp64 row statistics"},
        "us_per_call": round(us, 3), "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
        "metric_bytes": metric_bytes,
        "preroll_calls": t["preroll_calls"], "warmup_calls": t["warmup_calls"],
        "timing": ("median over replays of a graph of `steps` calls (--graph)" if args.graph else
                   "HIP events around exactly `steps` eager back-to-back calls, queued behind untimed filler work "
                   "so that no host launch gap falls inside; after the pre-roll and warm-up"),
        "path_us": other, "hot_us_cache_resident": None if hot is None else round(hot, 3),
        "replays": t.get("replays"),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": algo_bytes,
                     "kernel": "row_kernel" if chosen == "one" else "flat_kernel+row_kernel"},
        "device": torch.cuda.get_device_name(0),
        "arch": torch.cuda.get_device_properties(0).gcnArchName,
        **run_meta(torch, arrms),
    }
    if not args.no_probe and not wl.fp8:
        lib = load_probe()
        if lib is not None:
            pt = time_probe(torch, lib, wl, sets, args.steps, args.warmup, args.replays)
            pu = pt["us_per_call"]
            # the kernel timed the same way as the probe (inside graphs)
            kcalls = [lambda st, d=d: call(arrms, wl, d, wl.flags | path_flags[chosen], st) for d in sets.sets]
            ku, ku_min = time_graph_calls(torch, kcalls, max(args.steps, 64))
            line["graph_us_per_call"] = round(ku, 3)
            rd_bytes = (wl.R + 1) * wl.M * wl.H * e
            wr_bytes = 2 * wl.M * wl.H * e
            line["probe"] = {"kind": "data movement only: R+1 input and 2 output streams per row, no arithmetic",
                             "us_per_call": round(pu, 3), "min_us": round(pt["min_us"], 3),
                             "achieved": round(algo_bytes / (pu * 1e-6) / 1e9, 2), **pt["launch"],
                             "read_only": {"us_per_call": round(pt["read_only_us"], 3),
                                           "achieved": round(rd_bytes / (pt["read_only_us"] * 1e-6) / 1e9, 2)},
                             "write_only": {"us_per_call": round(pt["write_only_us"], 3),
                                            "achieved": round(wr_bytes / (pt["write_only_us"] * 1e-6) / 1e9, 2)},
                             "timing": "inside graphs, like graph_us_per_call"}
            line["probe_us"] = round(pu, 3)
            line["frac_of_probe"] = round(pu / ku, 4)
    del sets
    torch.cuda.empty_cache()
    if not args.no_workloads:
        wres = {}
        for w2 in [wlmod.SMALL, wlmod.HEADLINE, wlmod.FP8_GEMMA, wlmod.WIDE_R8, *wlmod.TAILS, wlmod.TAIL_FP32]:
            if w2.name == wl.name:
                continue
            wres[w2.name] = time_workload(torch, arrms, w2, ("one", "two"), args.steps, args.warmup)
        line["workloads"] = wres
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
