"""bench.py's output contract.

CPU: asking for more than one GPU exits with status 2 and says why.
GPU: a short run prints one JSON line with the contract's keys and types,
including the `roofline` and `cpu_baseline` objects.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    run = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert run.returncode == 2
    assert "one GPU" in run.stderr


@pytest.mark.gpu
def test_short_run_prints_the_contract_line():
    cmd = [sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--no-decode", "--no-noncausal", "--no-backward",
           "--no-sweep", "--no-generation", "--cpu-sample-tokens", "1024"]
    run = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr[-2000:]
    lines = [l for l in run.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, run.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "tokens/s"
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["config"]["workload"] == "causal_bf16_b2h8n131072"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] <= 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and isinstance(c["sample"], str)
