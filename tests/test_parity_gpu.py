"""Parity of the HIP path (through the C ABI) with the CPU oracle, on a GPU.

Every case runs the oracle and the HIP kernels on the same seeded host inputs
and compares them element by element over the whole output (the oracle is
plain C and finishes even the 2800 x 6144 and 2048 x 7168 x R=8 workloads in
seconds). Outputs are poisoned with NaN bytes before each call so that an
element the kernels fail to write shows up.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from all_reduce_residual_rank_amd import workloads as wlmod
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from all_reduce_residual_rank_amd import arrms
else:  # pragma: no cover - collected on CPU only with -m gpu deselected
    arrms = None

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")
PATHS = {"one": 16, "two": 32}   # FORCE_ONE_STAGE / FORCE_TWO_STAGE


def _case(wl, seed, paths, **kw):
    """Oracle once, then the HIP path once per named path; all compared to the oracle."""
    if isinstance(paths, str):
        paths = (paths,)
    xs, res, w = wlmod.make_inputs(wl, seed=seed)
    want = gu.run_oracle(wl, xs, res, w)
    for path in paths:
        print(f"case {wl.name} R={wl.R} M={wl.M} H={wl.H} {wl.dtype} flags={wl.flags} "
              f"seed={seed} path={path}", flush=True)
        got = gu.run_hip(wl, xs, res, w, extra_flags=PATHS[path], **kw)
        gu.compare(got, want, wl.dtype, label=f"{wl.name}/s{seed}/{path}")


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("wl", wlmod.ALL, ids=lambda w: w.name)
def test_workloads_seed0(wl, path):
    _case(wl, 0, path)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
@pytest.mark.parametrize("wl", wlmod.ALL, ids=lambda w: w.name)
def test_workloads_more_seeds(wl, seed):
    _case(wl, seed, "one")


def test_fp8_with_mirror_matches_quant_of_mirror():
    _case(wlmod.FP8_GEMMA.with_(mirror=True), 0, ("one", "two"))


@pytest.mark.parametrize("wl", [wlmod.HEADLINE, wlmod.FP8_GEMMA.with_(mirror=True), wlmod.TAIL_FP32,
                                wlmod.TAILS[2]], ids=lambda w: w.name)
def test_fast_branches_equal_exact_branches(wl):
    xs, res, w = wlmod.make_inputs(wl, seed=7)
    fast = gu.run_hip(wl, xs, res, w)
    exact = gu.run_hip(wl, xs, res, w, extra_flags=arrms.EXACT_ONLY)
    for k in fast:
        if fast[k] is not None:
            assert np.array_equal(fast[k], exact[k]), k


@pytest.mark.parametrize("wl", [wlmod.SMALL, wlmod.HEADLINE, wlmod.FP8_GEMMA.with_(mirror=True),
                                wlmod.WIDE_R8, wlmod.TAIL_FP32] + wlmod.TAILS,
                         ids=lambda w: w.name)
def test_one_stage_equals_two_stage_bitwise(wl):
    xs, res, w = wlmod.make_inputs(wl, seed=3)
    a = gu.run_hip(wl, xs, res, w, extra_flags=PATHS["one"])
    b = gu.run_hip(wl, xs, res, w, extra_flags=PATHS["two"])
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("path", ["one", "two"])
def test_inplace_residual(path):
    wl = wlmod.TAILS[4]
    xs, res, w = wlmod.make_inputs(wl, seed=1)
    want = gu.run_oracle(wl, xs, res, w)
    got = gu.run_hip(wl, xs, res, w, inplace=True, extra_flags=PATHS[path])
    gu.compare(got, want, wl.dtype, label="inplace")


def _page_shape_cases():
    g = json.load(open(GOLDEN))
    cases = []
    for M, H in g["fused_kernel_check_tp4"]["rows_hidden"]:
        cases.append(("tp4", 4, M, H))
    for M, H in g["fused_kernel_check_tp2"]["rows_hidden"]:
        cases.append(("tp2", 2, M, H))
    for M, H in g["fp8_identity"]["rows_hidden"]:
        cases.append(("fp8", 4, M, H))
    for M in g["upstream_2880"]["rows"]:
        cases.append(("up2880", 4, M, 2880))
    for M in g["decode_m"]["rows"]:
        cases.append(("decode", 8, M, 6144))
    return cases


@pytest.mark.parametrize("case", _page_shape_cases(), ids=lambda c: f"{c[0]}-R{c[1]}-{c[2]}x{c[3]}")
def test_page_shapes(case):
    kind, R, M, H = case
    variants = [dict(dtype="bf16"), dict(dtype="fp16", gemma=True, w_mean=0.0)]
    if kind == "fp8":
        variants = [dict(dtype="bf16", fp8=True, mirror=True),
                    dict(dtype="fp16", fp8=True, mirror=True, gemma=True, w_mean=0.0)]
    for v in variants:
        _case(wlmod.Workload(f"{kind}", R=R, M=M, H=H, **v), 11, ("one", "two"))


@pytest.mark.parametrize("R", range(1, 9))
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_every_rank_count(R, dtype):
    wl = wlmod.Workload("rsweep", R=R, M=37, H=1024 if dtype != "fp32" else 512, dtype=dtype,
                        fp8=dtype != "fp32", mirror=True, row_scale=(0.1, 10.0))
    _case(wl, R, ("one", "two"))


# every R at a size whose rows are all resident at once with inputs above
# 16 MiB: the narrow load window, where residual_out is written after the
# reduction (R = 1, 7, 8) or after the row's other outputs (R = 2 to 6); the T
# output in bf16 and per-token FP8 (with the mirror) in fp16
@pytest.mark.parametrize("R", range(1, 9))
@pytest.mark.parametrize("kind", ["bf16_t", "fp16_fp8"])
def test_every_rank_count_resident_rows(R, kind):
    if kind == "bf16_t":
        wl = wlmod.Workload("rsweep_resident", R=R, M=1024, H=6144, row_scale=(0.1, 10.0))
    else:
        wl = wlmod.Workload("rsweep_resident_fp8", R=R, M=1024, H=6144, dtype="fp16", gemma=True, fp8=True,
                            mirror=True, w_mean=0.0)
    _case(wl, 40 + R, ("one", "two"))


# launches of 6 or more input streams that run in several rounds of blocks
# (occupancy capped at 16 waves per compute unit)
@pytest.mark.parametrize("R", [5, 6, 7])
def test_capped_occupancy_rows(R):
    wl = wlmod.Workload("capped", R=R, M=2048, H=7168, eps=1e-5)
    _case(wl, 50 + R, ("one",))


@pytest.mark.parametrize("H", [8, 16, 64, 136, 504, 520, 1016, 3072, 5120, 8200, 16384])
def test_hidden_sizes_and_tails(H):
    wl = wlmod.Workload("hsweep", R=3, M=19, H=H, dtype="bf16", fp8=True, mirror=True)
    _case(wl, 5, ("one", "two"))


@pytest.mark.parametrize("H", [8188, 8192, 12284, 16380, 16384])
def test_widest_fp32_rows(H):
    # fp32 rows up to the hidden cap (64 KiB, 4096 packs: blocks of 1024 threads),
    # ragged and exact
    wl = wlmod.Workload("fp32wide", R=4, M=11, H=H, dtype="fp32", gemma=True, w_mean=0.0)
    _case(wl, 9, ("one", "two"))


@pytest.mark.parametrize("R,M", [(8, 7), (1, 600), (3, 300)])
def test_fp32_hidden_cap_rank_counts(R, M):
    # the widest fp32 rows at the extreme rank counts (R = 8 takes more packs per
    # thread than the register budget asks for), and launches of several hundred rows
    wl = wlmod.Workload("fp32cap", R=R, M=M, H=16384, dtype="fp32")
    _case(wl, 11 + R, ("one", "two"))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_exact_integer_sums(dtype):
    # the exact-integer generator of PR #5807's reproducer at its tail neighbours
    for M in (1023, 1024, 1025):
        H = 512
        xs = wlmod.exact_integer_inputs(4, M, H, seed=100 + M, dtype=dtype)
        wl = wlmod.Workload("exint", R=4, M=M, H=H, dtype=dtype)
        res = torch.zeros(M, H, dtype=gu.TORCH_T[dtype])
        w = torch.ones(H, dtype=gu.TORCH_T[dtype])
        want = gu.run_oracle(wl, xs, res, w)
        idx = np.arange(M * H).reshape(M, H)
        exact = sum(((idx * (r + 1) + (100 + M) * (r + 3)) % 31) - 15 for r in range(4))
        for path in ("one", "two"):
            got = gu.run_hip(wl, xs, res, w, extra_flags=PATHS[path])
            gu.compare(got, want, dtype, label=f"exint{M}")
            assert np.array_equal(gu._values(got["residual_out"], dtype), exact.astype(np.float64))


def test_special_values():
    # zero rows (FP8 scale 0, signed zeros), a row spanning a wide dynamic range
    # (FP8 subnormal codes, fp16 subnormal outputs), and a row hitting saturation.
    M, H = 6, 1024
    for dtype in ("bf16", "fp16"):
        T = gu.TORCH_T[dtype]
        g = torch.Generator().manual_seed(0)
        base = torch.randn(M, H, generator=g)
        x0 = base.clone()
        x0[0] = -0.0
        x0[1] = 0.0
        x0[2] = base[2] * torch.logspace(-7, 3, H)
        x0[3, :] = 1e-3
        x0[3, 17] = 3e4 if dtype == "fp16" else 3e30
        xs = [x0.to(T)] + [torch.zeros(M, H).to(T) for _ in range(2)]
        xs[1][0] = -0.0
        xs[2][0] = -0.0
        res = torch.zeros(M, H).to(T)
        res[0] = -0.0
        w = (torch.randn(H, generator=g) * 0.1 + 1.0).to(T)
        wl = wlmod.Workload("special", R=3, M=M, H=H, dtype=dtype, fp8=True, mirror=True)
        want = gu.run_oracle(wl, xs, res, w)
        assert want["scale"][0] == 0 and want["scale"][1] == 0
        for path in ("one", "two"):
            for extra in (0, arrms.EXACT_ONLY):
                got = gu.run_hip(wl, xs, res, w, extra_flags=PATHS[path] | extra)
                gu.compare(got, want, dtype, label=f"special-{dtype}-{path}")
                assert np.array_equal(got["fp8"], want["fp8"])


def test_deterministic_repeat():
    wl = wlmod.HEADLINE
    xs, res, w = wlmod.make_inputs(wl, seed=0)
    a = gu.run_hip(wl, xs, res, w)
    b = gu.run_hip(wl, xs, res, w)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k])


def test_graph_replay_with_changing_inputs():
    # Capture one call per path in a HIP graph, then replay with new inputs copied
    # into the captured buffers and NaN-poisoned outputs, checking every replay.
    dev = torch.device("cuda")
    wl = wlmod.Workload("graph", R=4, M=300, H=2880, dtype="fp16", gemma=True, fp8=True, mirror=True,
                        w_mean=0.0)
    arrms.arrms_reserve_staging(0)
    xs0, res0, w0 = wlmod.make_inputs(wl, seed=0)
    xd = [x.to(dev) for x in xs0]
    rd, wd = res0.to(dev), w0.to(dev)
    outs = {}
    graphs = {}
    for path in ("one", "two"):
        o = {"out": torch.empty(wl.M, wl.H, dtype=torch.float16, device=dev),
             "rout": torch.empty(wl.M, wl.H, dtype=torch.float16, device=dev),
             "q": torch.empty(wl.M, wl.H, dtype=torch.uint8, device=dev),
             "sc": torch.empty(wl.M, dtype=torch.float32, device=dev)}
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            arrms.arrms_fused(xd, rd, wd, o["out"], o["rout"], o["q"], o["sc"], eps=wl.eps,
                              flags=wl.flags | PATHS[path], stream=s)
        torch.cuda.current_stream().wait_stream(s)
        outs[path], graphs[path] = o, g
    for step in range(3):
        xs, res, w = wlmod.make_inputs(wl, seed=10 + step)
        for d, h in zip(xd, xs):
            d.copy_(h)
        rd.copy_(res)
        wd.copy_(w)
        want = gu.run_oracle(wl, xs, res, w)
        for path in ("one", "two"):
            o = outs[path]
            for t in o.values():
                gu.poison_(t)
            torch.cuda.synchronize()
            graphs[path].replay()
            torch.cuda.synchronize()
            got = {"out": gu.host_bits(o["out"]), "residual_out": gu.host_bits(o["rout"]),
                   "fp8": gu.host_bits(o["q"]), "scale": gu.host_bits(o["sc"])}
            gu.compare(got, want, "fp16", label=f"graph-{path}-{step}")


def test_two_stage_in_capture_without_staging_is_refused():
    dev = torch.device("cuda")
    torch.cuda.synchronize()
    arrms.arrms_release_staging()
    assert arrms.arrms_staging_bytes() == 0
    M, H = 8, 512
    xs = [torch.randn(M, H, device=dev).to(torch.bfloat16) for _ in range(2)]
    res = torch.randn(M, H, device=dev).to(torch.bfloat16)
    w = torch.ones(H, device=dev, dtype=torch.bfloat16)
    out = torch.empty_like(res)
    rout = torch.empty_like(res)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    dummy = torch.zeros(1, device=dev)
    with torch.cuda.graph(g, stream=s):
        dummy.add_(1)
        rc = arrms.arrms_fused_raw(xs, 2, res, w, out, rout, None, None, M, H, 1e-6,
                                   arrms.FORCE_TWO_STAGE, s.cuda_stream)
    assert rc == arrms.ERR_NO_STAGING
    # outside capture the same call reserves staging lazily and succeeds
    rc = arrms.arrms_fused_raw(xs, 2, res, w, out, rout, None, None, M, H, 1e-6,
                               arrms.FORCE_TWO_STAGE, torch.cuda.current_stream().cuda_stream)
    assert rc == arrms.OK
    torch.cuda.synchronize()
    assert arrms.arrms_staging_bytes() == arrms.DEFAULT_STAGING_BYTES


def test_graph_survives_staging_growth():
    # a graph captured on the two-stage path holds the staging address it was
    # captured with; growing the staging afterwards retires that buffer instead
    # of freeing it, so the graph keeps replaying correctly (and the eager calls
    # in between, which take the new buffer, stay correct too)
    dev = torch.device("cuda")
    torch.cuda.synchronize()
    arrms.arrms_release_staging()
    wl = wlmod.Workload("regrow", R=3, M=64, H=2880, dtype="bf16")
    arrms.arrms_reserve_staging(9 * 2880 * 2)  # 9 rows: the captured call runs 8 chunks
    small = arrms.arrms_staging_bytes()
    xs, res, w = wlmod.make_inputs(wl, seed=41)
    want = gu.run_oracle(wl, xs, res, w)
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    out = torch.empty(wl.M, wl.H, dtype=torch.bfloat16, device=dev)
    rout = torch.empty_like(out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        arrms.arrms_fused(xd, rd, wd, out, rout, eps=wl.eps, flags=wl.flags | PATHS["two"], stream=s)
    torch.cuda.synchronize()
    try:
        for step in range(3):
            # grow the staging (a new buffer each time; the old ones are retired)
            arrms.arrms_reserve_staging(small * (step + 2))
            assert arrms.arrms_staging_bytes() == small * (step + 2)
            eager = gu.run_hip(wl, xs, res, w, extra_flags=PATHS["two"])
            gu.compare(eager, want, wl.dtype, label=f"eager-after-growth-{step}")
            gu.poison_(out)
            gu.poison_(rout)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = {"out": gu.host_bits(out), "residual_out": gu.host_bits(rout), "fp8": None, "scale": None}
            gu.compare(got, want, wl.dtype, label=f"replay-after-growth-{step}")
    finally:
        del g
        torch.cuda.synchronize()
        arrms.arrms_release_staging()


def test_small_staging_forces_many_chunks():
    # a staging buffer of a few rows exercises the chunk loop (and its row offsets)
    torch.cuda.synchronize()
    arrms.arrms_release_staging()
    arrms.arrms_reserve_staging(7 * 2880 * 2 + 100)
    wl = wlmod.Workload("chunks", R=4, M=121, H=2880, dtype="fp16", fp8=True, mirror=True)
    try:
        _case(wl, 2, "two")
    finally:
        torch.cuda.synchronize()
        arrms.arrms_release_staging()


def _run_config(wl, xs, res, w, flags, ppt, tpr, rpb, blocks, window):
    dev = torch.device("cuda")
    T = gu.TORCH_T[wl.dtype]
    M, H = res.shape
    fp8 = bool(flags & arrms.FP8)
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    out = gu.poison_(torch.empty(M, H, dtype=T, device=dev)) if (wl.mirror or not fp8) else None
    rout = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    q = gu.poison_(torch.empty(M, H, dtype=torch.uint8, device=dev)) if fp8 else None
    sc = gu.poison_(torch.empty(M, dtype=torch.float32, device=dev)) if fp8 else None
    arrms.arrms_fused_config(xd, rd, wd, out, rout, q, sc, eps=wl.eps, flags=flags, ppt=ppt, tpr=tpr,
                             rows_per_block=rpb, blocks=blocks, load_window=window, M=M, H=H)
    torch.cuda.synchronize()
    return {"out": None if out is None else gu.host_bits(out), "residual_out": gu.host_bits(rout),
            "fp8": None if q is None else gu.host_bits(q), "scale": None if sc is None else gu.host_bits(sc)}


# (ppt, tpr, rows_per_block, blocks, load_window): one row group per block,
# row loops over a few blocks (every block takes several rows in turn),
# several row groups side by side per block, wide one-pack blocks, and the
# three phase-1 load windows
SHAPES = [(0, 0, 0, 0, 0), (0, 0, 0, 7, 0), (0, 0, 0, 64, 1), (1, 0, 0, 5, 2), (2, 0, 0, 33, 1),
          (4, 0, 0, 3, 2), (2, 0, 2, 11, 2), (1, 0, 0, 1, 1), (4, 0, 0, 0, 1), (4, 0, 0, 0, 2),
          (2, 0, 0, 0, 1), (1, 0, 0, 0, 2), (4, 0, 0, 0, 3), (3, 0, 0, 9, 3), (2, 0, 2, 0, 3),
          (1, 0, 0, 0, 3)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "ppt%d-tpr%d-rpb%d-b%d-w%d" % s)
@pytest.mark.parametrize("wl", [
    wlmod.Workload("cfg_bf16", R=4, M=131, H=6144, row_scale=(0.1, 10.0)),
    wlmod.Workload("cfg_fp16_fp8", R=3, M=77, H=2880, dtype="fp16", gemma=True, fp8=True, mirror=True,
                   w_mean=0.0),
    wlmod.Workload("cfg_r8_7168", R=8, M=45, H=7168, eps=1e-5),
    wlmod.Workload("cfg_fp32", R=2, M=60, H=512, dtype="fp32"),
], ids=lambda w: w.name)
def test_launch_shapes_match_oracle(wl, shape):
    ppt, tpr, rpb, blocks, window = shape
    P = wl.H * wl.esize // 16
    if ppt:
        need = -(-P // ppt)
        need = -(-need // 64) * 64
        if need * max(rpb, 1) > (1024 if ppt == 1 else 512):
            pytest.skip("shape cannot cover this row")
    xs, res, w = wlmod.make_inputs(wl, seed=12)
    want = gu.run_oracle(wl, xs, res, w)
    print(f"case {wl.name} shape={shape}", flush=True)
    got = _run_config(wl, xs, res, w, wl.flags | PATHS["one"], ppt, tpr, rpb, blocks, window)
    gu.compare(got, want, wl.dtype, label=f"{wl.name}/{shape}")


def test_concurrent_streams():
    # one-stage calls keep no state between calls: calls of different shapes,
    # dtypes and entry points enqueued on three streams at once must each give
    # the oracle's bits
    dev = torch.device("cuda")
    wa = wlmod.Workload("conc_a", R=4, M=300, H=6144, row_scale=(0.1, 10.0))
    wb = wlmod.Workload("conc_b", R=2, M=200, H=2880, dtype="fp16", gemma=True, fp8=True, mirror=True,
                        w_mean=0.0)
    ins = {}
    for wl, seed in ((wa, 41), (wb, 42)):
        xs, res, w = wlmod.make_inputs(wl, seed=seed)
        ins[wl.name] = (xs, res, w, [x.to(dev) for x in xs], res.to(dev), w.to(dev))
    sx = wlmod.make_sum_inputs(3, 1 << 20, 43, "bf16", sigma=1.0)
    sxd = [x.to(dev) for x in sx]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    print("concurrent streams: 2 x (bf16 300x6144, fp16 gemma FP8 200x2880, sum 1M)", flush=True)
    for rep in range(2):
        xs, res, w, xd, rd, wd = ins["conc_a"]
        oa = gu.poison_(torch.empty(wa.M, wa.H, dtype=torch.bfloat16, device=dev))
        ra = gu.poison_(torch.empty(wa.M, wa.H, dtype=torch.bfloat16, device=dev))
        xs, res, w, xd2, rd2, wd2 = ins["conc_b"]
        ob = gu.poison_(torch.empty(wb.M, wb.H, dtype=torch.float16, device=dev))
        rb = gu.poison_(torch.empty(wb.M, wb.H, dtype=torch.float16, device=dev))
        qb = gu.poison_(torch.empty(wb.M, wb.H, dtype=torch.uint8, device=dev))
        sb = gu.poison_(torch.empty(wb.M, dtype=torch.float32, device=dev))
        so = gu.poison_(torch.empty(1 << 20, dtype=torch.bfloat16, device=dev))
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        arrms.arrms_fused(xd, rd, wd, oa, ra, eps=wa.eps, flags=wa.flags | PATHS["one"], stream=streams[0])
        arrms.arrms_fused(xd2, rd2, wd2, ob, rb, qb, sb, eps=wb.eps, flags=wb.flags | PATHS["one"],
                          stream=streams[1])
        arrms.arrms_allreduce_sum(sxd, so, flags=arrms.DTYPE_BF16, stream=streams[2])
        outs.append((oa, ra, ob, rb, qb, sb, so))
    torch.cuda.synchronize()
    xs, res, w = ins["conc_a"][:3]
    want_a = gu.run_oracle(wa, xs, res, w)
    xs, res, w = ins["conc_b"][:3]
    want_b = gu.run_oracle(wb, xs, res, w)
    want_s = oracle.rank_sum([gu.host_bits(x) for x in sx], wlmod.DT_CODE["bf16"])
    for rep, (oa, ra, ob, rb, qb, sb, so) in enumerate(outs):
        gu.compare({"out": gu.host_bits(oa), "residual_out": gu.host_bits(ra), "fp8": None, "scale": None},
                   want_a, "bf16", label=f"conc-a-{rep}")
        gu.compare({"out": gu.host_bits(ob), "residual_out": gu.host_bits(rb), "fp8": gu.host_bits(qb),
                    "scale": gu.host_bits(sb)}, want_b, "fp16", label=f"conc-b-{rep}")
        assert np.array_equal(gu.host_bits(so), want_s), f"conc-sum-{rep}"
