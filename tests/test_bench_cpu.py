"""CPU checks of the benchmark's host logic: the one-GPU rule, the
algorithmic bytes behind the roofline, and the summaries it writes from
rocprofv3 output (synthetic CSV files here; no GPU and no profiler)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from selective_state_space_ssm2d_amd.inputs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


# Compulsory bytes of one forward launch: x and delta read and y written once
# (E elements each), B and C read once (batch * d_state * H * W each, not once
# per channel), A (d_inner * d_state fp32) and D (d_inner fp32). Worked out by
# hand from each workload's sizes:
#   wsi_mil        655,360 * 12 + 81,920 * 8 + 8,192 + 512         =   8,528,384
#   vmamba_t_s1    19,267,584 * 6 + 1,605,632 * 4 + 12,288 + 768   = 122,041,088
#   grid14         9,633,792 * 12 + 200,704 * 8 + 49,152 + 3,072  = 117,263,360
#   gigapixel_wsi  25,165,824 * 12 + 3,145,728 * 8 + 8,192 + 512   = 327,164,416
EXPECTED_BYTES = {"wsi_mil": 8_528_384, "vmamba_t_s1": 122_041_088, "grid14": 117_263_360,
                  "gigapixel_wsi": 327_164_416}


@pytest.mark.parametrize("name", sorted(EXPECTED_BYTES))
def test_algorithmic_bytes(name):
    wl = next(w for w in WORKLOADS if w.name == name)
    assert bench.algorithmic_bytes(wl) == EXPECTED_BYTES[name]
    # an accumulating launch also reads y
    s = 2 if wl.dtype == "bf16" else 4
    assert bench.algorithmic_bytes(wl, accumulate=True) == EXPECTED_BYTES[name] + wl.elements * s


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


SCAN = "void ssm2d_impl::scan2d_fwd_kernel<float, 4, 2, 4, 8, true, 0>(ssm2d_impl::Params)"
COPY = "void at::native::copy_kernel<float>"


def test_pmc_summary_scales_by_the_copy(tmp_path):
    d = str(tmp_path)
    # per dispatch, counters may come in several rows (summed); the median
    # dispatch is taken; other kernels are ignored
    _write_counters(f"{d}/sf", [(1, SCAN, "FETCH_SIZE", 50), (1, SCAN, "FETCH_SIZE", 50), (2, SCAN, "FETCH_SIZE", 200),
                                (3, SCAN, "FETCH_SIZE", 300), (4, "other", "FETCH_SIZE", 1e9)])
    _write_counters(f"{d}/sw", [(1, SCAN, "WRITE_SIZE", 70), (2, SCAN, "WRITE_SIZE", 80), (3, SCAN, "WRITE_SIZE", 90)])
    # a 512 MiB copy: FETCH_SIZE reads half of it, WRITE_SIZE all of it (KiB)
    _write_counters(f"{d}/cf", [(1, COPY, "FETCH_SIZE", 256 * 1024)])
    _write_counters(f"{d}/cw", [(1, COPY, "WRITE_SIZE", 512 * 1024)])
    rec = bench.pmc_summary("gigapixel_wsi", f"{d}/sf", f"{d}/sw", f"{d}/cf", f"{d}/cw", copy_mb=512, out_dir=d)
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(200 * 1024 * 2.0)
    assert rec["write_bytes_per_launch"] == pytest.approx(80 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(200 * 2048 + 80 * 1024)
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
    with open(os.path.join(d, "traffic_gigapixel_wsi.json")) as f:
        assert json.load(f)["bytes_per_launch"] == pytest.approx(rec["bytes_per_launch"])


def test_counter_table_medians_and_fractions(tmp_path):
    d = str(tmp_path)
    _write_counters(f"{d}/a", [(1, SCAN, "SQ_INSTS_VALU", 10), (1, SCAN, "SQ_INSTS_VALU", 5),
                               (2, SCAN, "SQ_INSTS_VALU", 30), (3, SCAN, "SQ_INSTS_VALU", 20)])
    _write_counters(f"{d}/b", [(1, SCAN, "SQ_WAVE_CYCLES", 1000), (1, SCAN, "SQ_WAIT_ANY", 400),
                               (2, SCAN, "SQ_WAVE_CYCLES", 1000), (2, SCAN, "SQ_WAIT_ANY", 500),
                               (3, SCAN, "SQ_WAVE_CYCLES", 1000), (3, SCAN, "SQ_WAIT_ANY", 450),
                               (4, COPY, "SQ_WAIT_ANY", 1e9)])
    med = bench.counter_table("gigapixel_wsi", [f"{d}/a", f"{d}/b"], out_dir=d)
    assert med["SQ_INSTS_VALU"] == 20 and med["SQ_WAIT_ANY"] == 450 and med["SQ_WAVE_CYCLES"] == 1000
    text = open(os.path.join(d, "sq_counters_gigapixel_wsi.txt")).read()
    assert "SQ_WAIT_ANY | 0.450" in text
    assert "rocprofv3 --pmc" in text


def test_trace_summary_lists_kernels(tmp_path):
    d = str(tmp_path)
    os.makedirs(f"{d}/t")
    with open(f"{d}/t/trace_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow([SCAN, 25, 7250000, 290000.0, 281000, 310000, 98.9])
    bench.trace_summary("gigapixel_wsi", f"{d}/t", out_dir=d)
    lines = open(os.path.join(d, "kernel_stats_gigapixel_wsi.txt")).read().splitlines()
    assert lines[1].startswith("# command:") and "rocprofv3 --kernel-trace --stats" in lines[1]
    assert "ssm2d_impl::scan2d_fwd_kernel<float, 4, 2, 4, 8, true, 0> | 25 | 7250000 | 290000.0" in lines[4]
