"""In-tree build of libmoe.so (HIP, gfx950) with hipcc.

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(the -packed-fp32-ops target feature) and linked into one shared library next
to this file.  Run ``python -m routed_expert_streaming_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["abi.cpp", "router.hip", "ffn_gemv.hip", "ffn_decode.hip", "ffn_mfma.hip", "ffn_entry.hip", "cache.hip",
           "residual.hip", "noalloc.hip", "cpu_lane.cpp"]
# host-only C++ (no HIP), built with the host compiler: the CPU lane
HOST_SOURCES = {"cpu_lane.cpp"}

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CXX = shutil.which("g++") or "g++"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument"]
# Extra -D tuning knobs (e.g. MOE_EXTRA_DEFINES="MOE_STREAM_NT=1 MOE_GEMV_BLOCKS_IN_FLIGHT=8")
COMMON += [f"-D{d}" for d in os.environ.get("MOE_EXTRA_DEFINES", "").split() if d]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src in HOST_SOURCES:
        cmd = [CXX, "-O3", "-std=c++17", "-fPIC", "-pthread", "-ffp-contract=off", "-Wall", f"-I{INCLUDE}",
               "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{CXX} failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str | None = None) -> str:
    global BUILD_DIR
    target = out or LIB
    if out:
        BUILD_DIR = os.path.join(ROOT, "_build", os.path.basename(out) + ".d")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = target + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, target)
    if verbose:
        print(f"built {target}")
    return target


if __name__ == "__main__":
    build(verbose=True, out=sys.argv[1] if len(sys.argv) > 1 else None)
    sys.exit(0)
