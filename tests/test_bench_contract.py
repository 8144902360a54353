"""bench.py's command-line contract.

On the CPU: more than one GPU is refused with exit status 2 and a message, before anything touches a
GPU, and every workload the help lists has its default step and warm-up counts.  On the GPU: a short
default run prints exactly one JSON line with the fields the contract names (metric, value, unit,
n_gpus, steps, warmup, ms_per_step, roofline with bound / achieved / peak / unit / frac / traffic,
cpu_baseline with value / unit / cores / kind / sample)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    for extra_env in ({}, {"WORLD_SIZE": "2"}):
        env = dict(os.environ, **extra_env)
        args = [sys.executable, BENCH] + ([] if extra_env else ["--gpus", "2"])
        res = subprocess.run(args, capture_output=True, text=True, env=env, timeout=120)
        assert res.returncode == 2, res.stderr
        assert "one GPU" in res.stderr
        assert res.stdout.strip() == ""


def test_every_workload_has_defaults():
    sys.path.insert(0, ROOT)
    import bench
    for name in bench.WORKLOAD_CLASSES:
        assert name in bench.WARMUP_DEFAULT, name
        assert bench.WORKLOAD_CLASSES[name].name == name


@pytest.mark.gpu
def test_default_run_prints_one_contract_line():
    res = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "2"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
    for k in ("prefill90min", "decode16", "ceiling"):
        assert k in d, k
    assert d["prefill90min"]["unit"] == "TFLOP/s" and 0 < d["prefill90min"]["frac"] < 1
    assert d["decode16"]["unit"] == "GB/s" and 0 < d["decode16"]["frac"] < 1
    assert d["ceiling"]["copy_gbs"] > 0 and d["ceiling"]["page_read_gbs"] > 0
    c = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "affinity_cores", "cpu_model", "kind", "sample", "prefill_tflops"):
        assert k in c, k
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
