"""The benchmark's data-movement probe (probe/libstream_probe.so) on the host: it
exports its four entry points and rejects shapes it does not take before any
launch. Device pointers are fake addresses that are never dereferenced; every
call below returns from the argument checks (or from rows == 0)."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "probe", "libstream_probe.so")
ENTRY_POINTS = ("probe_rows", "probe_rows_split", "probe_rows_read", "probe_rows_write")
FAKE = 1 << 40

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="probe not built (python __graft_entry__.py)")


@pytest.fixture(scope="module")
def lib():
    import bench  # loads the probe with its argument types
    return bench.load_probe()


def _ptrs(n):
    vp = ctypes.c_void_p
    return (vp * n)(*[FAKE + (i << 32) for i in range(n)])


def test_exports():
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    names = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    assert set(ENTRY_POINTS) <= names


def test_mixed_probe_rejects_bad_shapes(lib):
    ok = dict(nin=5, nout=2, rows=0, row_bytes=12288, ppt=4, tpr=192, window=2)

    def call(**kw):
        a = {**ok, **kw}
        return lib.probe_rows(_ptrs(a["nin"]), a["nin"], _ptrs(2), a["nout"], a["rows"], a["row_bytes"], a["ppt"],
                              a["tpr"], a["window"], None)

    assert call() == 0
    for bad in (dict(nin=1), dict(nin=10), dict(nout=1), dict(rows=-1), dict(row_bytes=12290), dict(ppt=5),
                dict(tpr=96), dict(tpr=128), dict(window=4)):
        assert call(**bad) == -1, bad


def test_one_sided_probes_reject_bad_shapes(lib):
    def rd(nin=5, sink=FAKE, rows=0, row_bytes=12288, ppt=4, tpr=192, window=2):
        return lib.probe_rows_read(_ptrs(nin), nin, sink, rows, row_bytes, ppt, tpr, window, None)

    def wr(nout=2, rows=0, row_bytes=12288, ppt=4, tpr=192):
        return lib.probe_rows_write(_ptrs(2), nout, rows, row_bytes, ppt, tpr, None)

    assert rd() == 0 and wr() == 0
    for bad in (dict(nin=1), dict(nin=10), dict(sink=None), dict(rows=-1), dict(row_bytes=8), dict(ppt=0),
                dict(tpr=1088), dict(tpr=128), dict(window=5)):
        assert rd(**bad) == -1, bad
    for bad in (dict(nout=3), dict(rows=-1), dict(row_bytes=24), dict(ppt=5), dict(tpr=64)):
        assert wr(**bad) == -1, bad
