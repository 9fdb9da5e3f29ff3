"""bench.py's byte accounting and traffic lookup (CPU only).

The metric counts (R+2)*M*H*2 + H*2 bytes per call; the roofline counts what
the path must move: the R inputs and the residual read, out and residual_out
written, the weight (per-token FP8: codes and fp32 scales instead of out).
The expected values below are those figures for the five workloads, worked
out by hand from the sizes (R=4 1024 x 6144 bf16: 6 * 1024 * 6144 * 2 + 6144
* 2 = 75,509,760 metric bytes, and so on).
"""
import json
import os

import pytest

import bench
from all_reduce_residual_rank_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("wl,metric,algo", [
    (W.SMALL, 1_191_936, 1_388_544),
    (W.HEADLINE, 75_509_760, 88_092_672),
    (W.FP8_GEMMA, 206_450_688, 223_665_088),
    (W.WIDE_R8, 293_615_616, 322_975_744),
])
def test_bytes_per_call(wl, metric, algo):
    assert bench.metric_bytes_of(wl) == metric
    assert bench.algo_bytes_of(wl) == algo


def test_tail_rows_metric_bytes():
    # the tail/decode sweep: (R+2)*M*H*e + H*e
    want = {(1, 2880): 40_320, (64, 2880): 2_217_600, (121, 2880): 4_187_520, (1023, 512): 6_286_336,
            (1024, 512): 6_292_480, (1025, 512): 6_298_624}
    for wl in W.TAILS:
        assert bench.metric_bytes_of(wl) == want[(wl.M, wl.H)]
    assert bench.metric_bytes_of(W.TAIL_FP32) == 12_597_248


def test_rotating_sets_exceed_the_infinity_cache():
    for wl in (W.HEADLINE, W.FP8_GEMMA, W.WIDE_R8):
        n = bench.nsets_for(wl, 256)
        assert n * (wl.R + 3) * wl.M * wl.H * wl.esize >= 512 << 20


def test_traffic_table_is_keyed_on_a_library_build():
    db = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert db
    for key, e in db.items():
        assert len(e["library_build"]) == 16 and int(e["library_build"], 16) >= 0, key
        assert e["hbm_bytes_per_launch"] > 0, key
        assert os.path.exists(os.path.join(ROOT, "profiles", e["summary"])), key
    # the lookup answers only for the build it was measured on
    e = db["r4_m1024_h6144_bf16_rowscale/one"]
    assert bench.load_traffic("r4_m1024_h6144_bf16_rowscale", "one", e["library_build"]) == e["hbm_bytes_per_launch"]
    assert bench.load_traffic("r4_m1024_h6144_bf16_rowscale", "one", "0" * 16) is None
    assert bench.load_traffic("r4_m1024_h6144_bf16_rowscale", "one", None) is None
    # counters within 1 % of the algorithmic bytes: no re-reads
    assert abs(e["hbm_bytes_per_launch"] / bench.algo_bytes_of(W.HEADLINE) - 1) < 0.01
