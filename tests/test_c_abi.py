"""The library as a plain C program sees it: tests/c_abi/host_calls.c is
compiled with gcc against include/ddpsim.h, linked to libddpsim.so and run
(host-side entry points only, no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "bucketed_gradient_all_ddp_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(LIB_DIR, "libddpsim.so")):
        pytest.skip("needs gcc and the built library")
    exe = str(tmp_path_factory.mktemp("cabi") / "host_calls")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "host_calls.c"), "-o", exe,
                    "-L", LIB_DIR, "-lddpsim", f"-Wl,-rpath,{LIB_DIR}",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], check=True)
    return exe


def test_c_caller_plans_prices_and_reports_errors(program, oracle):
    out = subprocess.run([program], capture_output=True, text=True, timeout=60, check=True)
    lines = out.stdout.splitlines()
    assert lines[0] == "params 148 buckets 13"
    from bucketed_gradient_all_ddp_amd import workloads as W
    sizes = [W.numel(s) for _, s in W.gpt2_small_params()]
    want = oracle.bucket_plan(sizes, 4, 25 << 20, 1 << 20)
    for b in range(13):
        assert lines[1 + b] == (f"bucket {b} size {len(want.bucket_params(b))} "
                                f"numel {want.bucket_numel(b)}")
    # the overlapped step time against the oracle's model (25 MiB buckets
    # throughout, so the oracle's grouping is the plan's)
    from oracle import costmodel as cm
    n = len(sizes)
    grads = [(sizes[i] * 4, (n - i) * 1e-3) for i in reversed(range(n))]
    step, exposed = cm.ddp_step_time(grads, bucket_cap=25 << 20, p=8, alpha=10e-6,
                                     beta=1 / 50e9)
    word, got_step, got_exposed = lines[14].split()
    assert word == "overlap"
    assert (float(got_step), float(got_exposed)) == (step, exposed)
    # 4.4 MB is the page's crossover: recursive doubling below, ring above
    assert lines[15] == "choose 4.3MB 1 4.5MB 0"
    assert lines[16] == "error 1 invalid argument"


@pytest.mark.gpu
def test_c_caller_all_reduces_on_the_gpu_without_torch(oracle, tmp_path):
    """tests/c_abi/device_allreduce.c allocates with hipMalloc, calls
    ring_allreduce_sim on its own stream and dumps inputs and outputs; the
    outputs must be the oracle's bits. It then runs the bf16 ring through
    ring_allreduce_sim_noalloc eagerly and from a captured HIP graph."""
    import numpy as np

    exe = str(tmp_path / "device_allreduce")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "device_allreduce.c"), "-o", exe,
                    "-L", LIB_DIR, "-lddpsim", f"-Wl,-rpath,{LIB_DIR}",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], check=True)
    out = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    p, n = 4, 1000003
    ins = np.fromfile(tmp_path / "inputs.bin", dtype=np.float32).reshape(p, n)
    got = np.fromfile(tmp_path / "outputs.bin", dtype=np.float32).reshape(p, n)
    want, log = oracle.ring_allreduce([ins[r] for r in range(p)], avg="world")
    for r in range(p):
        assert np.array_equal(got[r].view(np.uint32), want[r].view(np.uint32)), r
    C = -(-n // p)
    assert out.stdout.split() == ["steps", "6", "messages", str(len(log)),
                                  "bytes_sent_per_rank", str(2 * (p - 1) * C * 4)]
    # the no-allocation entry point on bf16 with the step-by-step ring:
    # eager, captured in a HIP graph, and that graph replayed on its own
    # results
    nb = 100003
    bins = {k: np.fromfile(tmp_path / f"bf16_{k}.bin", dtype=np.uint16).reshape(p, nb)
            for k in ("inputs", "eager", "graph1", "graph2")}
    want, _ = oracle.ring_allreduce([bins["inputs"][r] for r in range(p)], avg="world",
                                    want_log=False)
    for r in range(p):
        assert np.array_equal(bins["eager"][r], want[r]), f"eager rank {r}"
        assert np.array_equal(bins["graph1"][r], want[r]), f"replay 1 rank {r}"
    again, _ = oracle.ring_allreduce([bins["graph1"][r] for r in range(p)], avg="world",
                                     want_log=False)
    for r in range(p):
        assert np.array_equal(bins["graph2"][r], again[r]), f"replay 2 rank {r}"
