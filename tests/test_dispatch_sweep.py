"""The automatic dispatch against the committed launch-shape sweep (CPU only).

profiles/dispatch_sweep.csv holds, for a grid of rows x hidden x ranks and two
kinds of call (bf16 with the T output; fp16 gemma_norm with the per-token FP8
output), the measured us per call of every one-stage launch shape (packs per
thread x load window), of the two-stage path and of the automatic choice, with
the device facts the library reported (its occupancy for the chosen shape and
the compute units). Two checks:

  * the rules as they stand reproduce the automatic choice recorded in each row
    (arrms_plan_launch, pure host, fed the recorded device facts), so the CSV
    describes the current rules;
  * at every point the automatic choice is within 2 % of the best variant
    measured, or within 0.15 us of it for latency-bound calls (a few us, where
    run-to-run noise alone is of that size). The chosen configuration is
    measured twice in each row group -- as the "auto" row and as the explicit
    variant of the same shape and window -- and the better of the two counts.

The table the library uses is generated from a separate training sweep
(profiles/dispatch_sweep_train.csv, gen_dispatch_table.py); this file checks
it against the validation sweep profiles/dispatch_sweep.csv, measured with
that table in the library.
"""
import csv
import os
from collections import defaultdict

import pytest

from all_reduce_residual_rank_amd import arrms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSV = os.path.join(ROOT, "profiles", "dispatch_sweep.csv")

KINDS = {"bf16": (arrms.DTYPE_BF16, 0), "fp16_fp8": (arrms.DTYPE_FP16 | arrms.GEMMA | arrms.FP8, 1)}
REL_TOL = 0.02
ABS_TOL_US = 0.15


def _points():
    pts = defaultdict(list)
    with open(CSV) as f:
        for row in csv.DictReader(f):
            pts[(row["kind"], int(row["R"]), int(row["M"]), int(row["H"]))].append(row)
    return pts


def test_sweep_covers_the_grid():
    pts = _points()
    Ms = {k[2] for k in pts}
    Hs = {k[3] for k in pts}
    Rs = {k[1] for k in pts}
    assert {1, 16, 64, 256, 1024, 2800, 4096} <= Ms
    assert {512, 2880, 4096, 6144, 7168, 8192} <= Hs
    assert {2, 4, 8} <= Rs
    assert {k[0] for k in pts} == set(KINDS)
    for key, rows in pts.items():
        variants = {r["variant"] for r in rows}
        assert "auto" in variants and "two" in variants, key
        assert any(v.startswith("ppt") for v in variants), key


def test_table_is_generated_from_the_training_sweep():
    import importlib.util
    gen = os.path.join(ROOT, "all_reduce_residual_rank_amd", "csrc", "gen_dispatch_table.py")
    spec = importlib.util.spec_from_file_location("gen_dispatch_table", gen)
    g = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(g)
    want = g.render(g.best_variants(g.DEFAULT_CSV), g.DEFAULT_CSV)
    assert open(g.OUT).read() == want


def test_rules_reproduce_the_recorded_choice():
    for (kind, R, M, H), rows in _points().items():
        flags, quant = KINDS[kind]
        auto = next(r for r in rows if r["variant"] == "auto")
        plan = arrms.arrms_plan_launch(M, H, R, flags & ~arrms.FP8, quant, False, int(auto["blocks_per_cu"]),
                                       int(auto["cus"]))
        got = (plan["path"], plan["ppt"], plan["tpr"], plan["window"], plan["cap16"])
        want = tuple(int(auto[k]) for k in ("auto_path", "auto_ppt", "auto_tpr", "auto_window", "auto_cap16"))
        assert got == want, (kind, R, M, H)


def test_auto_is_within_tolerance_of_the_best():
    worst = []
    for key, rows in _points().items():
        a = next(r for r in rows if r["variant"] == "auto")
        same = f"ppt{a['auto_ppt']}_w{a['auto_window']}" if a["auto_path"] == "1" else "two"
        auto = min(float(r["us_median"]) for r in rows if r["variant"] in ("auto", same))
        best_row = min((r for r in rows if r["variant"] != "auto"), key=lambda r: float(r["us_median"]))
        best = float(best_row["us_median"])
        if auto > max(best * (1 + REL_TOL), best + ABS_TOL_US):
            worst.append((key, auto, best, best_row["variant"]))
    assert not worst, worst
