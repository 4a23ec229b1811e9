"""The benchmark's output contract on the GPU: one short run of bench.py in a
child process, its one JSON line checked field by field."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_roofline(gpu_lib):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--stage-reps", "2",
           "--no-cpu-baseline", "--no-full-context", "--no-decode", "--no-stack"]
    print("running", " ".join(cmd), flush=True)
    run = subprocess.run(cmd, capture_output=True, text=True, timeout=100, cwd=ROOT)
    assert run.returncode == 0, run.stderr[-3000:]
    lines = [ln for ln in run.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, run.stdout[-2000:]
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["unit"] == "tokens/s" and out["higher_is_better"] is True and out["dtype"] == "bf16"
    assert out["config"]["workload"] == "qwen1p7b_32k"
    n = out["config"]["n"]
    assert out["value"] > 0 and out["ms_per_step"] > 0
    # value is prompt tokens over the timed step time (ms_per_step is rounded in the JSON)
    assert abs(out["value"] * out["ms_per_step"] / 1e3 / n - 1.0) < 5e-3
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert abs(roof["achieved"] - roof["flops_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e12) < 0.5
    assert roof["launches_timed"] == 3
    assert out["cpu_baseline"] is None  # switched off for this run
    for stage in ("prune", "rope_kv", "attn"):  # the step's own stages, in path order
        assert out["stages"][stage]["median_us"] > 0
    for stage in ("prune", "gate", "gate_select", "select", "gather", "rope_kv", "attn"):
        assert out["stages"][stage]["cold_us"] > 0
        assert out["stages"][stage]["us_back_to_back"] > 0
    assert out["stages"]["gather"]["back_to_back_cache"] == "cold"
    assert out["prune_entry"] == "tg_gate_select_gather"
    for key in ("gather_pct_hbm_peak", "gate_pct_hbm_peak", "rope_kv_pct_hbm_peak"):
        assert 0 < out[key] < 100, key
    assert out["pruning"]["select_plus_gather_us"] > 0 and out["pruning"]["prune_us"] > 0
    assert roof["avg_launch_us_back_to_back"] > 0 and 0 < roof["frac_back_to_back"] < 1
