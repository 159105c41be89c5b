"""The benchmark's JSON line on the GPU: every field the line promises,
with the roofline and CPU-baseline objects consistent with themselves."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_line():
    print("bench line: gigapixel_wsi, 3 steps", flush=True)
    r = subprocess.run([sys.executable, "bench.py", "--steps", "3", "--warmup", "1", "--cpu-seconds", "1"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "elements/s" and d["higher_is_better"] is True and d["dtype"] == "f32"
    assert d["config"]["workload"] == "gigapixel_wsi"
    elements = d["config"]["batch"] * d["config"]["d_inner"] * d["config"]["H"] * d["config"]["W"]
    assert d["value"] == pytest.approx(elements / (d["ms_per_step"] * 1e-3), rel=1e-6)
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    # the named bound of the scan: HBM, algorithmic bytes over the mean launch
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0.0 < roof["frac"] < 1.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    c = d["config"]
    abytes = elements * 12 + c["batch"] * c["d_state"] * c["H"] * c["W"] * 8 + c["d_inner"] * (c["d_state"] + 1) * 4
    assert roof["algorithmic_bytes"] == abytes
    assert roof["achieved"] == pytest.approx(abytes / (roof["kernel_ms_mean"] * 1e-3) / 1e9, rel=1e-6)
    assert roof["kernel_ms_mean"] <= d["ms_per_step"] * 1.05
    # secondary ALU view: 9 flops per (element, state) against the published fp32 peak
    alu = d["alu"]
    assert alu["peak"] == 157.3 and alu["unit"] == "TFLOP/s"
    assert alu["achieved"] == pytest.approx(elements * c["d_state"] * 9 / (roof["kernel_ms_mean"] * 1e-3) / 1e12,
                                            rel=1e-6)
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "elements/s" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["sample"]
