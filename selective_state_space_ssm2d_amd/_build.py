"""Build step for libssm2d.so (gfx950). Used by ``__graft_entry__.build()``."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ssm2d.hip")
LIB = os.path.join(PKG, "libssm2d.so")
INCLUDE = os.path.join(ROOT, "include")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC", "-shared",
]


def build(out_path: str = LIB) -> str:
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", INCLUDE, SRC, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    return out_path
