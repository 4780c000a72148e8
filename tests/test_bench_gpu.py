"""bench.py's one JSON line on the GPU: the keys, types and relations the
measurement contract fixes, from a short run of the default workload."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "5", "--cpu-budget", "1"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    print(f"[bench] {lines[0][:300]}", flush=True)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["dtype"] == "f16"
    assert d["config"]["workload"] == "sweep_s8192_d128"
    flops = 4 * 2 * 16 * 8192 * 8192 * 128 / 2
    assert d["config"]["flops_per_step"] == flops
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2516.6
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0 < rf["achieved"] < rf["peak"]
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    ps = d["parity_sample"]
    assert ps["max_abs_o"] <= ps["tol_o"] and ps["lse_rel"] <= ps["tol_lse_rel"]
