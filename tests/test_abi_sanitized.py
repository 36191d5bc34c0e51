"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/host/abi_check.cpp`` links the argument checks and the chunk planner
(``flce_api.cpp``, ``flce_plan.cpp``) with stubs in place of the kernels and of
the two HIP runtime calls that read the status word, builds them with g++
and ``-fsanitize=address,undefined`` (host code only: nothing here is GPU
code), and runs: every rejection case of the entry points (each must return
its code and launch nothing), valid calls (each launches once, with a plan
that fits its workspace), the status reader, every error string, and a seeded
sweep of 20000 planner calls over shapes and budgets (the plan invariants,
and the workspace size agreeing with the plan).  Any sanitizer report aborts
the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_gemm_amd", "csrc")


def test_abi_host_code_is_clean_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ and the ROCm headers are needed")
    exe = str(tmp_path / "abi_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "abi_check.cpp"), os.path.join(CSRC, "flce_api.cpp"),
           os.path.join(CSRC, "flce_plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-4000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "0 failed checks" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
