"""Build step for libssm2d.so (gfx950). Used by ``__graft_entry__.build()``.

The kernel instances are split over several translation units (one per input
type and lane layout) that hipcc compiles in parallel; the objects are then
linked into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# one translation unit per (input type, lane layout or mode)
_VARIANTS = ("g4", "g8", "flipw", "vfirst", "flipw_vfirst", "acc", "flipw_acc", "vfirst_acc", "flipw_vfirst_acc",
             "states", "bwd", "bwd_edges", "states_flipw", "bwd_ltr", "bwd_ltr_edges", "gate", "gate_flipw", "fast",
             "rowc", "rowc_vfirst", "states_rowc", "states_flipw_rowc", "bwd_rowc", "bwd_edges_rowc", "bwd_ltr_rowc",
             "bwd_ltr_edges_rowc", "narrow")
SOURCES = ["ssm2d.hip"] + [f"scan2d_{t}_{v}.hip" for t in ("f32", "bf16") for v in _VARIANTS]
LIB = os.path.join(PKG, "libssm2d.so")
INCLUDE = os.path.join(ROOT, "include")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-lane LDS counter updates stay single instructions
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-fPIC",
]


def build(out_path: str = LIB) -> str:
    with tempfile.TemporaryDirectory(prefix="ssm2d_build_") as tmp:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = ["hipcc", *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        errors = []
        for src, pr in procs:
            out, _ = pr.communicate()
            if pr.returncode != 0:
                errors.append(f"{src}:\n{out}")
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp_out = out_path + ".tmp"
        cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
        os.replace(tmp_out, out_path)
    return out_path
