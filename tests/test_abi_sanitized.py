"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): api.cpp is built with gcc and the sanitizers, the kernel launches
are replaced by stubs that launch nothing, and a driver calls every entry
point with a seeded sweep of valid and invalid arguments (sizes, strides,
flags, alignments, overlaps, quant forms, launch shapes). Any sanitizer
report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "all_reduce_residual_rank_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip/hip_runtime.h"),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_is_sanitizer_clean(tmp_path):
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}"]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "kernel_stubs.cpp"),
                os.path.join(HERE, "abi_sweep.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["g++", *flags, "-c", src, "-o", obj], check=True, capture_output=True, text=True)
        objs.append(obj)
    exe = str(tmp_path / "abi_sweep")
    subprocess.run(["g++", *flags, *objs, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe, "60000"], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-3000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-3000:]
    assert "calls 60000" in report


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_staging_bookkeeping(tmp_path):
    """Growing the staging buffer retires the old one (kept allocated for graphs
    captured earlier); release frees each buffer exactly once."""
    exe = str(tmp_path / "staging_test")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", f"-I{CSRC}", os.path.join(HERE, "staging_test.cpp"),
                    "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "staging ok" in r.stdout
