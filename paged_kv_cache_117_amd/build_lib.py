"""Build libpa.so in-tree for gfx950 (``python -m paged_kv_cache_117_amd.build_lib``).

HIP sources are compiled with hipcc for gfx950 with packed-fp32 instructions
disabled; the host-only block manager and error plumbing with g++.  Objects
go to ``_build/`` at the repository root; the library lands next to this
file as ``libpa.so`` (written to a temporary name, then renamed).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa.so")

HIP_SOURCES = ["decode.hip", "decode_mfma.hip", "decode_api.hip", "cache_ops.hip", "prefill.hip", "prefill_api.hip",
               "probe.hip"]
CPP_SOURCES = ["block_manager.cpp", "sha256.cpp", "errors.cpp"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs rather than AGPRs: the decode kernel reads its
    # 4-register score tile straight back, and one register file keeps the
    # 16-bit GQA<=4 kernel within 128 registers (4 waves per SIMD).
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = True, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = max(1, min(jobs, 16))
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".hip.o"))
        cmds.append([HIPCC, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    # --no-undefined: a missing symbol (say, a kernel whose host-side launch
    # stub was not emitted) fails here instead of when the library loads
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    print(LIB)
