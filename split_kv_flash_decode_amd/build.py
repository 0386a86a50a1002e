"""Build the HIP library libskv.so in-tree for gfx950 with hipcc.

    python -m split_kv_flash_decode_amd.build [--jobs N]

Each source compiles to its own object in parallel, then one link step makes
``split_kv_flash_decode_amd/libskv.so``. The per-kernel register, LDS and
spill report that the compiler prints (-Rpass-analysis=kernel-resource-usage)
is kept next to the library in ``_build/resource_usage.txt``.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libskv.so")

ARCH = "gfx950"
HIP_SOURCES = ["skv_mfma.hip", "skv_valu.hip", "skv_combine.hip", "skv_plan.hip", "skv_noalloc.hip",
               "skv_ceiling.hip"]
CPP_SOURCES = ["skv_host.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Packed FP32 instructions are kept out of every device binary.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Rpass-analysis=kernel-resource-usage"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *DEVICE, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        # plain host C++ (no HIP in it): the system compiler
        cmd = [shutil.which("g++") or "g++", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CPP_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    report = "\n".join(
        line for _, err in results for line in err.splitlines()
        if "remark" in line or "Function Name" in line or "VGPRs" in line or "Spill" in line
        or "LDS" in line or "Occupancy" in line or "SGPRs" in line or "ScratchSize" in line)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(report + "\n")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
