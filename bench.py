"""Benchmark of the 2D selective scan forward on one MI355X.

One step = one ssm2d_scan_fwd call over one batch of the workload (inputs
resident in HBM). Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workload (default): the giga-pixel WSI grid, batch 1, d_inner 128, d_state 16,
H x W = 384 x 512, fp32, 60 % blob-shaped pad cells. Inputs are seeded and
synthetic. Several copies of the inputs are cycled so that the footprint of
consecutive steps exceeds the 256 MB Infinity Cache: every step reads HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# Plain fp32 VALU issue rate (no packed fp32): 256 CU x 4 SIMD x 16 lanes x
# 2.4 GHz = 39.3e12 slots/s; an FMA slot is 2 flops -> 78.6 TFLOP/s.
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2.4e9 * 2 / 1e12
# Algorithmic ALU work per (element, state): 2 mul + 3 FMA + 1 exp2, and exp2
# issues at half rate on gfx950 (2 slots), so 7 slots = 14 FMA-equivalent flops.
SLOTS_PER_ELEM_STATE = 7

METRIC = "2D-scan elements/s (B·D·H·W) + % of MI355X peak HBM GB/s"


def algorithmic_bytes(wl) -> int:
    s = 2 if wl.dtype == "bf16" else 4
    E = wl.elements
    return E * 3 * s + wl.batch * wl.d_state * wl.H * wl.W * 2 * s + wl.d_inner * wl.d_state * 4 + wl.d_inner * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gigapixel_wsi")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-maps", type=int, default=0, help="oracle sample size in (b,d) maps (0 = all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import selective_state_space_ssm2d_amd as pkg
    from selective_state_space_ssm2d_amd.inputs import WORKLOADS, make_inputs

    wl = {w.name: w for w in WORKLOADS}[args.workload]
    if not os.path.exists(pkg.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    pkg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = make_inputs(wl, seed=0)
    keys = ("x", "delta", "A", "B", "C", "D")

    def upload():
        out = []
        for k in keys:
            if wl.dtype == "bf16" and k in ("x", "delta", "B", "C"):
                out.append(torch.from_numpy(t[k + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16))
            else:
                out.append(torch.from_numpy(np.ascontiguousarray(t[k])).to(dev))
        return out

    abytes = algorithmic_bytes(wl)
    ncopies = max(2, int(np.ceil(768e6 / abytes)))
    sets = [upload() for _ in range(ncopies)]
    ys = [torch.empty_like(s[0]) for s in sets]

    stream = torch.cuda.current_stream()
    for w in range(args.warmup):
        k = w % ncopies
        pkg.scan_fwd(*sets[k], y=ys[k])
    pkg.sync_check()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        k = s % ncopies
        starts[s].record(stream)
        pkg.scan_fwd(*sets[k], y=ys[k])
        ends[s].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pkg.sync_check()
    kern_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    ms_step = wall * 1e3 / args.steps
    E = wl.elements
    value = E / (ms_step * 1e-3)
    kmean = float(np.mean(kern_ms))
    gbs = abytes / (kmean * 1e-3) / 1e9
    flops = E * wl.d_state * SLOTS_PER_ELEM_STATE * 2
    tflops = flops / (kmean * 1e-3) / 1e12

    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            traffic = json.load(f).get("bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        if not os.path.exists(oracle.LIB_PATH):
            oracle.build()
        nmaps = wl.batch * wl.d_inner
        sel = np.arange(nmaps if args.cpu_maps <= 0 else min(args.cpu_maps, nmaps))
        threads = oracle.max_threads()
        c0 = time.perf_counter()
        oracle.fwd(*(t[k] for k in keys), maps=sel)
        cw = time.perf_counter() - c0
        cpu = {"value": sel.size * wl.H * wl.W / cw, "unit": "elements/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{sel.size} of {nmaps} (b,d) maps of {wl.name}, fp64, {cw:.2f} s wall"}

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and pad structure of the workload, no dataset)",
        "config": {"workload": wl.name, "batch": wl.batch, "d_inner": wl.d_inner, "d_state": wl.d_state,
                   "H": wl.H, "W": wl.W, "pad": wl.pad, "pad_cells": wl.pad_cells,
                   "input_copies_cycled": ncopies},
        "roofline": {"bound": "alu", "achieved": tflops, "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / ALU_PEAK_TFLOPS, "traffic": traffic,
                     "kernel": "scan2d_fwd_kernel", "kernel_ms_mean": kmean,
                     "kernel_ms_median": float(np.median(kern_ms)), "kernel_ms_min": float(np.min(kern_ms))},
        "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": abytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
