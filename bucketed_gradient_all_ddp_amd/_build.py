"""Build libddpsim.so (the HIP library behind the C ABI in include/ddpsim.h).

Every source is compiled for gfx950 only, in-tree, with:
  -fhip-fp32-correctly-rounded-divide-sqrt   the averaging division is IEEE
  -fno-gpu-flush-denormals-to-zero           subnormal sums are kept
  -ffp-contract=off                          no fused multiply-add
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 math
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libddpsim.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["host.cpp", "plan.cpp", "allreduce.hip", "collectives.hip", "flatten.hip",
           "bucket_allreduce.hip", "reducer.cpp", "schedules.hip",
           "coalesced.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
    "-ffp-contract=off", "-fno-fast-math",
]
DEVICE = [
    f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def compile_commands(build_dir=BUILD_DIR, defines=()):
    cmds = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append(([HIPCC, *COMMON, *DEVICE, *[f"-D{d}" for d in defines], *lang,
                      "-c", path, "-o", obj], obj))
    return cmds


def build(verbose: bool = False, out: str = LIB_PATH, build_dir: str = BUILD_DIR,
          defines=()) -> str:
    """Compile every source (always) and link libddpsim.so (by default into
    the package). `defines` are extra -D tuning macros."""
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for cmd, obj in compile_commands(build_dir, defines):
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), cmd, obj))
    objs = []
    for proc, cmd, obj in procs:
        _, err = proc.communicate()
        # the host pass does not know the device-only feature flag: harmless
        for line in err.splitlines():
            if "packed-fp32-ops' is not a recognized feature" not in line:
                print(line, file=sys.stderr)
        if proc.returncode != 0:
            raise RuntimeError("compile failed: " + " ".join(cmd))
        objs.append(obj)
    tmp = out + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
