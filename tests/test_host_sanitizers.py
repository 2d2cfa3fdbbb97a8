"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the planner, the piece-table builder, the coalescing planner, the
overlap model and the argument checks, driven by tests/c_abi/host_sanitize.cpp
over 1,500 random plans. The host sources are rebuilt instrumented (host pass
only); the kernels' objects come from the ordinary build."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bucketed_gradient_all_ddp_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
KERNEL_OBJS = ["allreduce.hip.o", "collectives.hip.o", "bucket_allreduce.hip.o",
               "schedules.hip.o", "coalesced.hip.o", "flatten.hip.o"]


def test_host_code_is_clean_under_sanitizers(tmp_path):
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJS]
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and all(map(os.path.exists, objs))):
        pytest.skip("needs hipcc, clang++ and the library's build objects")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    sources = [os.path.join(CSRC, f) for f in ("host.cpp", "plan.cpp", "reducer.cpp")]
    sources.append(os.path.join(ROOT, "tests", "c_abi", "host_sanitize.cpp"))
    procs, outs = [], []
    for src in sources:
        out = str(tmp_path / (os.path.basename(src) + ".o"))
        outs.append(out)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", src, "-o", out],
                                      stderr=subprocess.PIPE, text=True))
    for proc in procs:
        _, err = proc.communicate(timeout=300)
        assert proc.returncode == 0, err[-2000:]
    exe = str(tmp_path / "host_sanitize")
    subprocess.run([CLANG, "-fsanitize=address,undefined", *outs, *objs,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe], check=True)
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert r.stdout.startswith("ok ") and "runtime error" not in r.stderr, r.stderr[-3000:]
