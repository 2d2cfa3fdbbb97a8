"""bench.py's output contract: one JSON line with the fields the driver
reads, a refusal of more than one GPU, and the traffic figure tied to the
kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_defaults_finish_within_minutes(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.gpus == 1 and a.steps == 20 and a.warmup == 5
    assert a.workload == "gpt2-small-p8"


def test_traffic_figure_follows_the_sources(monkeypatch):
    m = bench.MEASURED_TRAFFIC["bucket_allreduce_kernel"]
    assert bench.measured_traffic("bucket_allreduce_kernel") in (None, m["bytes_per_launch"])
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, "bucket_allreduce_kernel",
                        {"bytes_per_launch": 123, "sources_sha256": "0" * 64})
    assert bench.measured_traffic("bucket_allreduce_kernel") is None
    sha = bench.sources_sha256("bucket_allreduce_kernel")
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, "bucket_allreduce_kernel",
                        {"bytes_per_launch": 123, "sources_sha256": sha})
    assert bench.measured_traffic("bucket_allreduce_kernel") == 123
    assert bench.measured_traffic("no_such_kernel") is None


@pytest.mark.gpu
def test_headline_line_has_the_contract_fields():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-compare", "--cpu-buckets", "1"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert "workload" in d["config"] and "model" not in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.3 < rf["frac"] < 1.0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert cb["host_cores"] == os.cpu_count() and "GPU's own input values" in cb["sample"]
    assert len(d["config"]["arena_base_mod_2MiB"]) == d["config"]["p"]
    pc = d["practical_ceiling"]
    assert 1000 < pc["copy_GBps"] < 8000
    assert abs(pc["headline_frac_of_copy"] - rf["achieved"] / pc["copy_GBps"]) < 1e-3
