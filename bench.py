"""Benchmark of the 2D selective scan forward on one MI355X.

One step = one ssm2d_scan_fwd call over one batch of the workload (inputs
resident in HBM). Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--variant V]

--variant times another direction / order through ssm2d_scan_fwd_ex instead:
flip_hw (from the lower-right corner), vfirst (vertical-first order), four_way
(sum of the four corner scans: four launches per step, the last three adding
into y), four_way_vfirst; or bwd, the backward pass (ssm2d_scan_bwd: the
stored-state forward, the adjoint scan and the channel sums per step).

Workload (default): the giga-pixel WSI grid, batch 1, d_inner 128, d_state 16,
H x W = 384 x 512, fp32, 60 % blob-shaped pad cells. Inputs are seeded and
synthetic. Several copies of the inputs are cycled so that the footprint of
consecutive steps exceeds the 256 MB Infinity Cache: every step reads HBM.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
PROFILES = os.path.join(ROOT, "profiles")

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# Secondary ALU view. The published fp32 vector peak is 157.3 TFLOP/s (256 CU
# x 4 SIMD x 16 lanes x 2.4 GHz x 2 flops per FMA x 2 for packed fp32); this
# library builds without packed fp32 instructions, so its issue ceiling is
# half that: 39.3e12 VALU slots/s, 78.6 TFLOP/s counting an FMA as 2 flops.
ALU_PEAK_TFLOPS = 157.3
ALU_ISSUE_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
# Algorithmic work per (element, state): 1 exp2, 2 multiplies and 3 FMAs:
# 6 VALU instructions (each counted as one issue slot), 9 flops (exp 1,
# multiply 1, FMA 2).
SLOTS_PER_ELEM_STATE = 6
FLOPS_PER_ELEM_STATE = 9
# Backward per (element, state): the forward's 6 to recompute the states, then
# 21 for the adjoint: Abar (1 mul + exp2 = 2), u (1), g_h and its carry (2),
# the carried g_hh (2), hh (1), g_a Abar (4), g_hh B (1), d delta (2), dx (1),
# dB and dC terms (2), dA (1), and the sums over channels for dB, dC (2).
SLOTS_PER_ELEM_STATE_BWD = 6 + 21

METRIC = "2D-scan elements/s (B·D·H·W) + % of MI355X peak HBM GB/s"


def algorithmic_bytes(wl, accumulate=False) -> int:
    """Compulsory HBM bytes of one launch: x, delta, B, C, A, D read, y written
    (and read too, when the launch adds into y)."""
    s = 2 if wl.dtype == "bf16" else 4
    E = wl.elements
    return (E * (4 if accumulate else 3) * s + wl.batch * wl.d_state * wl.H * wl.W * 2 * s
            + wl.d_inner * wl.d_state * 4 + wl.d_inner * 4)


def algorithmic_bytes_bwd(wl) -> int:
    """Compulsory HBM bytes of the backward: x, delta, dy, B, C, A, D read;
    dx, d delta, dB, dC, dA, dD written (the stored states are not counted)."""
    s = 2 if wl.dtype == "bf16" else 4
    bnhw = wl.batch * wl.d_state * wl.H * wl.W
    return wl.elements * 5 * s + bnhw * 4 * s + 2 * (wl.d_inner * wl.d_state * 4 + wl.d_inner * 4)


# variant -> (ssm2d_scan_fwd_ex keywords, launches per step); None: ssm2d_scan_fwd
VARIANTS = {
    "fwd": (None, 1),
    "flip_hw": (dict(flip_h=True, flip_w=True), 1),
    "vfirst": (dict(vertical_first=True), 1),
    "four_way": (dict(four_way=True), 4),
    "four_way_vfirst": (dict(four_way=True, vertical_first=True), 4),
    "bwd": ("bwd", 3),
}


def _tag(workload: str, variant: str) -> str:
    return workload if variant == "fwd" else f"{workload}_{variant}"


KERNEL_SRC_DIR = os.path.join(ROOT, "selective_state_space_ssm2d_amd", "csrc")


def kernel_source_hash() -> str:
    """Hash of the library's HIP sources (counter summaries are only valid for
    the kernel they were taken on)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SRC_DIR)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(KERNEL_SRC_DIR, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def copy_probe(mb: int, steps: int) -> None:
    """A plain device-to-device copy of known size, for calibrating the
    FETCH_SIZE / WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch

    n = mb * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mb": mb, "steps": steps}))


# The scan kernels: the general one and the two-rows-per-step forward of tall maps.
SCAN_KERNELS = ("scan2d_fwd_kernel", "scan2d_fast_kernel", "scan2d_narrow_kernel")


def is_scan_kernel(name: str) -> bool:
    return any(k in name for k in SCAN_KERNELS)


def kernel_name(wl, variant: str) -> str:
    """The scan kernel(s) a step of the workload launches, as the library plans
    them (ssm2d_fwd_kernels): the two-rows-per-step forward, the general
    kernel, the whole-row kernel for narrow maps, or several joined by '+'
    (a four-corner sum can use two)."""
    import selective_state_space_ssm2d_amd as pkg

    kw, _ = VARIANTS[variant]
    if kw == "bwd":
        return "scan2d_fwd_kernel"  # the stored-state and adjoint passes
    fast, general, narrow = pkg.fwd_kernels(wl.batch, wl.d_inner, wl.d_state, wl.H, wl.W, bf16=wl.dtype == "bf16",
                                            **(kw or {}))
    names = ((["scan2d_fast_kernel"] if fast else []) + (["scan2d_fwd_kernel"] if general else [])
             + (["scan2d_narrow_kernel"] if narrow else []))
    return "+".join(names)


def _pmc_per_dispatch(run_dir: str, counter: str, name_part):
    """Median per dispatch of a counter over the kernels whose name contains
    name_part (a string, or a tuple of alternatives)."""
    parts = (name_part,) if isinstance(name_part, str) else tuple(name_part)
    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if any(q in r["Kernel_Name"] for q in parts) and r["Counter_Name"] == counter:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} under {run_dir}")
    v = sorted(vals.values())
    return v[len(v) // 2]  # median over dispatches


def pmc_summary(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                copy_mb: int, variant: str = "fwd", out_dir: str = PROFILES) -> dict:
    """Turns four rocprofv3 --pmc runs (scan FETCH_SIZE, scan WRITE_SIZE, copy
    FETCH_SIZE, copy WRITE_SIZE; KiB per dispatch) into calibrated HBM bytes
    per launch of the scan kernel: profiles/traffic_<workload>[_<variant>].json."""
    copy_bytes = copy_mb * 1024 * 1024
    cf = _pmc_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copy") * 1024.0
    cw = _pmc_per_dispatch(copy_write_dir, "WRITE_SIZE", "copy") * 1024.0
    sf = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", SCAN_KERNELS) * 1024.0
    sw = _pmc_per_dispatch(write_dir, "WRITE_SIZE", SCAN_KERNELS) * 1024.0
    kf, kw = copy_bytes / cf, copy_bytes / cw
    rec = {
        "workload": workload,
        "variant": variant,
        "kernel": " / ".join(SCAN_KERNELS),
        "kernel_source_sha256_16": kernel_source_hash(),
        "copy_probe_bytes": copy_bytes,
        "copy_fetch_counter_bytes": cf, "copy_write_counter_bytes": cw,
        "fetch_scale": kf, "write_scale": kw,
        "scan_fetch_counter_bytes": sf, "scan_write_counter_bytes": sw,
        "fetch_bytes_per_launch": sf * kf, "write_bytes_per_launch": sw * kw,
        "bytes_per_launch": sf * kf + sw * kw,
        "commands": ["cd /tmp && export TMPDIR=/tmp && cd <repo>"]
        + [PMC_SCAN_CMD.format(c=c, w=workload, v="" if variant == "fwd" else f" --variant {variant}")
           for c in ("FETCH_SIZE", "WRITE_SIZE")]
        + [PMC_COPY_CMD.format(c=c, mb=copy_mb) for c in ("FETCH_SIZE", "WRITE_SIZE")],
    }
    out = os.path.join(out_dir, f"traffic_{_tag(workload, variant)}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return rec


def cpu_baseline(wl, t, keys, seconds: float, kw=None):
    """Times the oracle as it is (fp64, OpenMP over maps, all host threads) on
    a bounded sample of the workload's (b, d) maps: calls over consecutive maps
    (all of them per call if a pass is short) repeat until about `seconds` of
    wall time have passed; a first untimed call over one map per thread sizes
    the calls."""
    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    nmaps = wl.batch * wl.d_inner
    threads = oracle.max_threads()
    ins = [np.ascontiguousarray(t[k], dtype=np.float64) for k in keys]  # the oracle's input type
    first = np.arange(min(threads, nmaps))
    c0 = time.perf_counter()
    oracle.fwd(*ins, maps=first, **(kw or {}))
    t_first = max(time.perf_counter() - c0, 1e-6)
    per_map = t_first / first.size
    chunk = nmaps if per_map * nmaps <= seconds / 2 else max(first.size, int(seconds / 4 / per_map))
    done, k = 0, 0
    c0 = time.perf_counter()
    while True:
        sel = (np.arange(chunk) + k) % nmaps
        oracle.fwd(*ins, maps=sel, **(kw or {}))
        done += sel.size
        k = (k + chunk) % nmaps
        cw = time.perf_counter() - c0
        if cw >= seconds:
            break
    n_el = done * wl.H * wl.W
    what = "map scans" if not kw else f"map scans ({', '.join(sorted(kw))})"
    return {"value": n_el / cw, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} (b,d) {what} ({nmaps} maps in the workload) of {wl.name} "
                      f"({wl.H}x{wl.W}, d_state {wl.d_state}), fp64, {cw:.1f} s wall on {threads} threads"}


def cpu_baseline_bwd(wl, t, keys, seconds: float):
    """Times the oracle's backward (fp64, OpenMP over batch entries) on the
    workload's first k channels (all batch entries and cells), k doubling from
    one until a call takes about `seconds` / 4, then repeated until `seconds`."""
    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    ins = [np.ascontiguousarray(t[k], dtype=np.float64) for k in keys]
    dy = np.random.default_rng(1).standard_normal(ins[0].shape)

    def call(k):
        sl = [ins[0][:, :k], ins[1][:, :k], ins[2][:k], ins[3], ins[4], ins[5][:k], dy[:, :k]]
        c0 = time.perf_counter()
        oracle.bwd(*sl)
        return time.perf_counter() - c0

    k = 1
    while True:
        dt = call(k)
        if dt >= seconds / 4 or k >= wl.d_inner:
            break
        k = min(wl.d_inner, 2 * k)
    done, total = 0, 0.0
    while total < seconds:
        total += call(k)
        done += k
    n_el = done * wl.batch * wl.H * wl.W
    threads = min(oracle.max_threads(), wl.batch)
    return {"value": n_el / total, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"backward of {done} channel maps in calls of {k} channels x {wl.batch} batch "
                      f"({wl.d_inner} channels in the workload) of {wl.name} ({wl.H}x{wl.W}, d_state {wl.d_state}), "
                      f"fp64, {total:.1f} s wall, OpenMP over the {wl.batch} batch entries"}


TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- "
             "python bench.py --workload {w} --steps {s} --warmup {wu} --no-cpu-baseline{v}")
# One counter per run (rocprofv3 does not split counters over passes).
PMC_SCAN_CMD = ("timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d <dir> -o pmc -- "
                "python bench.py --workload {w} --steps 5 --warmup 2 --no-cpu-baseline{v}")
PMC_COPY_CMD = ("timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d <dir> -o pmc -- "
                "python bench.py --copy-probe {mb} --steps 5")


def trace_summary(workload: str, run_dir: str, variant: str = "fwd", out_dir: str = PROFILES, steps: int = 20,
                  warmup: int = 5) -> None:
    """Writes profiles/kernel_stats_<workload>[_<variant>].txt from the kernel
    statistics of a rocprofv3 --kernel-trace --stats run of this benchmark
    (made with the given --steps and --warmup)."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    rows = list(csv.DictReader(open(files[0])))
    vopt = "" if variant == "fwd" else f" --variant {variant}"
    lines = [f"# rocprofv3 kernel statistics, workload {workload}, variant {variant}",
             f"# command: cd /tmp && export TMPDIR=/tmp && cd <repo> && {TRACE_CMD.format(w=workload, v=vopt, s=steps, wu=warmup)}",
             f"# kernel source sha256[:16] {kernel_source_hash()}",
             "# name | calls | total ns | average ns | min ns | max ns | percent"]
    for r in rows:
        short = r["Name"].replace("(anonymous namespace)::", "").removeprefix("void ").split("(")[0][:110]
        lines.append(f"{short} | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.1f} | "
                     f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f}")
    out = os.path.join(out_dir, f"kernel_stats_{_tag(workload, variant)}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SWEEP_CMD = "python bench.py --workload {w} --shape-sweep {spec}"
SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_BRANCH SQ_INSTS_VMEM SQ_INSTS_SMEM "
               "SQ_WAIT_INST_LDS",
               "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
               "SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_LDS SQ_BUSY_CYCLES")


def shape_sweep(wl, spec: str, reps: int = 20) -> None:
    """Mean kernel time of the forward over maps of the workload's batch,
    channels and states at other heights and widths ("HxW,HxW,..."), and for
    each width timed at two or more heights the least-squares fit
    t = fixed + H * per_row: a chain's pipeline start-up and drain against
    its steady row rate. Writes profiles/shape_sweep_<workload>.txt."""
    import torch

    import selective_state_space_ssm2d_amd as pkg
    from selective_state_space_ssm2d_amd.inputs import make_random_inputs

    pkg.load_library()
    dev = torch.device("cuda:0")
    shapes = [tuple(int(v) for v in hw.split("x")) for hw in spec.split(",")]
    lines = [f"# forward kernel time vs map shape, batch {wl.batch}, d_inner {wl.d_inner}, d_state {wl.d_state}, "
             f"{wl.dtype}; inputs: make_random_inputs(seed 0), no pad cells",
             f"# command: {SWEEP_CMD.format(w=wl.name, spec=spec)}",
             f"# kernel source sha256[:16] {kernel_source_hash()}",
             "# H | W | mean us | min us"]
    res = {}
    for H, W in shapes:
        t = make_random_inputs(wl.batch, wl.d_inner, wl.d_state, H, W, seed=0, dtype=wl.dtype)
        args = []
        for k in ("x", "delta", "A", "B", "C", "D"):
            if wl.dtype == "bf16" and k in ("x", "delta", "B", "C"):
                args.append(torch.from_numpy(t[k + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16))
            else:
                args.append(torch.from_numpy(np.ascontiguousarray(t[k])).to(dev))
        y = torch.empty_like(args[0])
        for _ in range(5):
            pkg.scan_fwd(*args, y=y)
        pkg.sync_check()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            pkg.scan_fwd(*args, y=y)
            b.record()
        torch.cuda.synchronize()
        pkg.sync_check()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        res[(H, W)] = float(us.mean())
        lines.append(f"{H} | {W} | {us.mean():.1f} | {us.min():.1f}")
        print(lines[-1], flush=True)
    lines.append("# W | fixed us | us per row (fit over the heights timed at that width)")
    for W in sorted({w for _, w in shapes}):
        hs = sorted(h for h, w in shapes if w == W)
        if len(hs) >= 2:
            slope, icpt = np.polyfit(hs, [res[(h, W)] for h in hs], 1)
            lines.append(f"{W} | {icpt:.1f} | {slope:.3f}")
    out = os.path.join(PROFILES, f"shape_sweep_{wl.name}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_table(workload: str, dirs, out_dir: str = PROFILES) -> dict:
    """Per-dispatch SQ counters of the scan kernel (median over dispatches)
    from rocprofv3 --pmc runs of this benchmark, one run per counter group:
    profiles/sq_counters_<workload>.txt."""
    lines = [f"# rocprofv3 SQ counters of the scan kernel, workload {workload} (median per dispatch; "
             "totals over the chip's waves)",
             f"# kernel source sha256[:16] {kernel_source_hash()}"]
    for grp in SQ_COUNTERS:
        lines.append("# command: cd /tmp && export TMPDIR=/tmp && cd <repo> && timeout -s KILL 90 rocprofv3 --pmc "
                     f"{grp} --output-format csv -d <dir> -o pmc -- python bench.py --workload {workload} "
                     "--steps 3 --warmup 1 --no-cpu-baseline")
    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            per = {}
            for r in csv.DictReader(open(f)):
                if is_scan_kernel(r["Kernel_Name"]):
                    key = (r["Dispatch_Id"], r["Counter_Name"])
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            for (_, name), v in per.items():
                vals.setdefault(name, []).append(v)
    if not vals:
        raise SystemExit("no scan kernel counter rows under " + " ".join(dirs))
    med = {k: sorted(v)[len(v) // 2] for k, v in vals.items()}
    for k in sorted(med):
        lines.append(f"{k} | {med[k]:.6g}")
    if "SQ_WAVE_CYCLES" in med:
        lines.append("# fractions of SQ_WAVE_CYCLES")
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS"):
            if k in med:
                lines.append(f"{k} | {med[k] / med['SQ_WAVE_CYCLES']:.3f}")
    out = os.path.join(out_dir, f"sq_counters_{workload}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return med


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gigapixel_wsi")
    ap.add_argument("--variant", default="fwd", choices=sorted(VARIANTS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target wall time of the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB MiB (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("SCAN_FETCH", "SCAN_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc output directories")
    ap.add_argument("--copy-mb", type=int, default=512)
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="write profiles/kernel_stats_<workload>.txt from a rocprofv3 --stats run "
                         "(pass the --steps and --warmup that run used)")
    ap.add_argument("--shape-sweep", metavar="HxW,...",
                    help="time the forward at other map heights and widths (fill against row rate)")
    ap.add_argument("--counter-table", nargs="+", metavar="PMC_DIR",
                    help="write profiles/sq_counters_<workload>.txt from rocprofv3 --pmc output directories")
    args = ap.parse_args()
    if args.counter_table:
        counter_table(args.workload, args.counter_table)
        return
    if args.trace_summary:
        trace_summary(args.workload, args.trace_summary, args.variant, steps=args.steps, warmup=args.warmup)
        return
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary, copy_mb=args.copy_mb, variant=args.variant)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe, max(1, args.steps))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import selective_state_space_ssm2d_amd as pkg
    from selective_state_space_ssm2d_amd.inputs import WORKLOADS, make_inputs

    wl = {w.name: w for w in WORKLOADS}[args.workload]
    if not os.path.exists(pkg.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    pkg.load_library()
    if args.shape_sweep:
        shape_sweep(wl, args.shape_sweep)
        return
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

    kw, launches = VARIANTS[args.variant]
    abytes = algorithmic_bytes(wl)
    ncopies = max(2, int(np.ceil(768e6 / abytes)))
    sets = [upload() for _ in range(ncopies)]
    ys = [torch.zeros_like(s[0]) for s in sets]
    if kw == "bwd":
        gen = torch.Generator(device="cpu").manual_seed(1)
        dys = [torch.randn(s[0].shape, generator=gen).to(dev, s[0].dtype) for s in sets]
        outs = [{"dx": torch.empty_like(s[0]), "ddelta": torch.empty_like(s[1]), "dA": torch.empty_like(s[2]),
                 "dB": torch.empty_like(s[3]), "dC": torch.empty_like(s[4]), "dD": torch.empty_like(s[5])}
                for s in sets]

    def step(k):
        if kw is None:
            pkg.scan_fwd(*sets[k], y=ys[k])
        elif kw == "bwd":
            pkg.scan_bwd(*sets[k], dys[k], out=outs[k])
        else:
            pkg.scan_fwd_ex(*sets[k], y=ys[k], **kw)

    stream = torch.cuda.current_stream()
    for w in range(args.warmup):
        step(w % ncopies)
    pkg.sync_check()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        k = s % ncopies
        starts[s].record(stream)
        step(k)
        ends[s].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pkg.sync_check()
    kern_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    ms_step = wall * 1e3 / args.steps
    E = wl.elements
    value = E / (ms_step * 1e-3)
    kmean = float(np.mean(kern_ms))        # one step: `launches` kernels back to back
    if kw == "bwd":
        # reads x, delta, B, C, dy, A, D; writes dx, d delta, dB, dC, dA, dD
        step_bytes = algorithmic_bytes_bwd(wl)
        slots = E * wl.d_state * SLOTS_PER_ELEM_STATE_BWD
        launches = 1  # roofline figures below are per step (three kernels)
    else:
        step_bytes = abytes if launches == 1 else abytes + (launches - 1) * algorithmic_bytes(wl, accumulate=True)
        slots = launches * E * wl.d_state * SLOTS_PER_ELEM_STATE
    gbs = step_bytes / (kmean * 1e-3) / 1e9
    tflops = slots * FLOPS_PER_ELEM_STATE / SLOTS_PER_ELEM_STATE / (kmean * 1e-3) / 1e12
    issue_floor_ms = slots / ALU_ISSUE_SLOTS_PER_S * 1e3

    # HBM bytes per launch from the committed counter summary, only while it
    # describes the kernel as it is now
    traffic = None
    tpath = os.path.join(PROFILES, f"traffic_{_tag(wl.name, args.variant)}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_bwd(wl, t, keys, args.cpu_seconds) if kw == "bwd" else \
            cpu_baseline(wl, t, keys, args.cpu_seconds, kw)

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
                   "input_copies_cycled": ncopies, "variant": args.variant, "launches_per_step": launches},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": step_bytes,
                     "kernel": kernel_name(wl, args.variant), "kernel_ms_mean": kmean / launches,
                     "kernel_ms_median": float(np.median(kern_ms)) / launches,
                     "kernel_ms_min": float(np.min(kern_ms)) / launches},
        "alu": {"achieved": tflops, "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / ALU_PEAK_TFLOPS,
                "flops_per_elem_state": FLOPS_PER_ELEM_STATE,
                "slots_per_elem_state": SLOTS_PER_ELEM_STATE_BWD if kw == "bwd" else SLOTS_PER_ELEM_STATE,
                "issue_floor_ms": issue_floor_ms / launches, "issue_frac": issue_floor_ms / kmean},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
