"""The C ABI from a plain C program (tests/native/abi_consumer.c): device
memory and a stream from the HIP runtime API, no PyTorch and no Python in the
process that calls libarrms.so. The program checks every output byte of three
cases (bf16: R=4 37x6144 plain; R=3 20x2880 gemma with FP8 and the mirror; R=8
5x7168 with FP8), both paths, against the CPU oracle, plus error returns, and
prints "abi_consumer ok". It is built by __graft_entry__.build()
(tests/native/build.py)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_consumer")


def test_plain_c_consumer_matches_oracle():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: build it with __graft_entry__.build() (tests/native/build.py)")
    print("native C consumer of libarrms.so", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_consumer ok" in r.stdout
    assert r.stdout.count("bit-identical to the oracle") == 6
