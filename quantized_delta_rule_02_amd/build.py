"""Builds libstepq.so (HIP kernels for gfx950 + the C++ runtime) in the package directory.

    python -m quantized_delta_rule_02_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libstepq.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
ARCH = os.environ.get("STEPQ_ARCH", "gfx950")

SOURCES = ["api.cpp", "planner.cpp", "kernels.hip", "probe.hip"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
              f"-I{os.path.join(os.path.dirname(HERE), 'include')}"]
    # packed FP32 (v_pk_*_f32) is disabled for all device code
    # IEEE mode off: no NaN arises on the step's path, and without it fmaxf/fminf compile to one
    # v_max/v_min instead of being preceded by canonicalizing copies of their operands
    device = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-munsafe-fp-atomics", "-mno-amdgpu-ieee", "-fno-honor-nans"]

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        path = os.path.join(CSRC, src)
        if src.endswith(".hip"):
            cmd = [hipcc, "-x", "hip"] + common + device + ["-c", path, "-o", obj]
        else:
            cmd = [hipcc] + common + ["-pthread", "-c", path, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            sys.stderr.write(res.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
