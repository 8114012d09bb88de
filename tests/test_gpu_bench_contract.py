"""bench.py's output contract on the GPU: one JSON line on stdout carrying the metric,
the value and its unit, the run's shape, the roofline record of the dominant kernel
and the CPU baseline, with figures that agree with each other.  A short run (two
token counts, two steps, a small CPU sample) keeps it to seconds of GPU time."""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    print("bench.py", *args, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines[:3]
    return json.loads(lines[0])


def test_bench_line_contract():
    out = run_bench("--m", "1,1024", "--steps", "2", "--warmup", "1", "--no-peaks",
                    "--cpu-sample-cols", "16")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["unit"] == "TOPS" and out["higher_is_better"] is True
    assert out["dtype"] == "int8" and out["data"] == "synthetic" and out["vs_baseline"] is None
    assert isinstance(out["config"]["workload"], str) and out["config"]["M"] == [1, 1024]
    assert out["value"] > 0 and out["ms_per_step"] > 0
    # value is the step's integer ops over the step time
    ops = sum(2.0 * M * N * K for M in (1, 1024) for (N, K) in out["config"]["layers"].values())
    ops *= len(out["config"]["abits"])
    assert abs(out["value"] - ops / (out["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * out["value"]
    roof = out["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and roof["peak"] in (5000.0, 8000.0)
    assert roof["unit"] in ("TOP/s", "GB/s")
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None          # counters belong to the default workload only
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["unit"] == "TOPS" and isinstance(cpu["sample"], str)
    # per-shape rows for every (M, abits, layer)
    assert len(out["shapes"]) == 2 * 2 * 4
    assert out["targets"]["hbm_frac_m_le_16"] > 0 and out["targets"]["int8_frac_m_ge_1024"] > 0


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
