"""The host side of the library (planner, plan serialization, argument checks) under AddressSanitizer
and UndefinedBehaviorSanitizer, with leak detection (no GPU: the kernel launchers are stubbed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_delta_rule_02_amd", "csrc")
HIP_LIB = "/opt/rocm/lib"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(HIP_LIB, "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library")
def test_plan_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_abi")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-pthread", os.path.join(ROOT, "tests", "host_plan_abi_driver.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(CSRC, "planner.cpp"), "-L" + HIP_LIB, "-lamdhip64", "-Wl,-rpath," + HIP_LIB, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "ok (0 failures)" in run.stdout
